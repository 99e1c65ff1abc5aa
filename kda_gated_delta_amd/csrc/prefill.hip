// KDA chunked prefill (export kda_chunk_prefill).
//
// Page "KDA Chunk Prefill on Ascend A3": section "Function and tensor
// contract" (shapes, GQA head mapping) and section "Mathematical definition"
// (Q/K L2 normalisation; the chunk construction G, L, A = solve(I+L,
// diag(beta)), W, U, Qg, Kg, Aqk; the carry Vnew = U - W S, O = Qg S + Aqk
// Vnew, S = exp(G_last) S + Kg^T Vnew; chunk size 64 with a zero-padded last
// chunk).
//
// Two kernels, split where the method splits: everything inside a chunk is
// independent of the state, so it runs chunk-parallel over the whole chip;
// only the carry is sequential.
//
// intra_kernel -- persistent: one 512-thread workgroup (8 waves) per compute
//   unit walks the (value head, chunk slot) work items with a grid stride,
//   prefetching the next item's inputs while it computes the current one.
//   Per chunk:
//     1. the raw q, k, g and beta, prefetched into registers while the
//        previous chunk was computed, are normalised (bit-exact routine
//        shared with kda_qk_l2norm; except for a workgroup's first item this
//        runs at the end of the previous item, behind its workspace
//        stores), scanned (G, kept in log2 units) and staged in LDS;
//     2. the gated L and Aqk, 16x16 blocks on MFMA;
//     3. T = (I+L)^-1 by blocked forward substitution in float32 (diagonal
//        blocks by substitution, off-diagonal blocks on fp32 MFMA), then
//        A = T diag(beta);
//     4. E = exp(G) k, Kg, Qg, exp(G_last) and W = A E (the split form
//        forms E, Kg and Qg during 3, beside the off-diagonal MFMA steps);
//   and the chunk's W, Qg, Kg^T, Aqk, A and exp(G_last) are written to the
//   workspace (66 KB per chunk and head, fp16 except exp(G_last)).
//
// inter_kernel<16> -- two 256-thread workgroups per (sequence, value head),
//   one per half of the state's 128 columns (the columns evolve
//   independently: column v of S only ever meets column v of the values),
//   placed on the same XCD so the second read of each chunk's workspace slot
//   hits L2.  Wave w of a half owns 16 columns and keeps that 128x16 slice of
//   S in registers as float32 for the whole sequence.  Chunk slots stream
//   through two LDS buffers (the next chunk is loaded while the current one
//   is computed).  Per chunk, on MFMA: U = A v and Vnew = U - W S accumulate
//   in float32 (U is never rounded), O^T = S^T Qg^T + Vnew^T Aqk^T, and
//   S = exp(G_last) S + Kg^T Vnew.
// inter_kernel<32> -- the same carry with one workgroup per unit, each wave
//   owning 32 columns (two 16-column tiles through the same operand reads).
//
// Two schedules of the split form.  Sequential: the chunk kernel over every
// item, then inter_kernel<16>.  Overlapped (equal-length sequences, 48 to
// CUs - 32 units, a workspace with room for ready flags): one chunk-kernel
// launch runs the first rs chunk rows (a row: one chunk of every unit) on
// every CU and the rest on the workgroups that stay, while
// inter_kernel<32>, on a second stream, takes the CUs of those that leave
// and polls a ready flag per slot.  Both give the same results bit for bit.
//
// Fused partition (export kda_chunk_prefill_fused): intra_kernel<true>, one
//   workgroup per (sequence, value head), runs steps 1-4 for that unit's
//   chunks in order and, in place of the workspace write, applies the carry
//   (the inter kernel's products, same order and precision) to a float32
//   state held by its 8 waves, 16 columns each, reading the operands from
//   LDS.  It saves the workspace round trip but puts the chunk-local work
//   on each unit's sequential path, so it pays off only with many units.
//
// Precision: every MFMA operand is fp16 with float32 accumulation, and the
// state is carried in float32.  fp16's 11-bit significand keeps the final
// state within a few 1e-4 (relative Frobenius) of the float64 recurrence
// even when beta = 1 and the gates barely decay, where bf16 operands drift
// past 1e-3.  The operands are bounded in magnitude (|A| <= 1, decay factors
// <= 1, normalised q and k), except v, the state and the split decay factors
// of diagonal blocks: v and the state must stay below 2^14 in magnitude, and
// a diagonal block whose split factors exceed 2^14 (gates below about -1.2
// per token) is computed with bf16 operands instead.
//
// Overflow-safe decay factors.  exp(G_i - G_j) for j <= i is <= 1, but it is
// needed inside dot products over the channel d, so it is split into a row
// factor and a column factor around a reference token r:
//   exp(G_i - G_j) = exp(G_i - G_r) * exp(G_r - G_j).
// For a 16x16 block below the diagonal, r is the first token of the row
// block, so both factors are <= 1.  For a diagonal block, r is the block's
// middle token, so each factor is at most exp of the decay accumulated over
// 8 tokens; if that exceeds 2^120 for any channel the block is computed
// pair by pair instead (exact, slow, only for extreme gates).  exp(-G) over a
// whole chunk is never formed.
//
// Workspace.  Chunk c of sequence n of value head hv lives in slot
// base(n) + c of head hv, with base(n) = floor(first_token(n) / 64) + n; the
// slots of consecutive sequences never overlap because a sequence of L
// tokens has ceil(L/64) <= floor(L/64) + 1 chunks.  A slot holds, in order:
//   W     fp16 [64][128]  channels in the permuted order below
//   Qg    fp16 [64][128]  channels permuted
//   Kg^T  fp16 [128][64]  tokens permuted
//   Aqk   fp16 [64][64]   tokens permuted
//   A     fp16 [64][64]   natural order
//   gamma fp32 [128]      exp(G_last)
// Within each row of the four matrices, the 16-byte piece p is stored at
// position p ^ (row & 7) (an XOR swizzle), so that sixteen lanes reading the
// same logical piece of sixteen consecutive rows hit distinct LDS banks once
// the slot is copied verbatim into LDS.
#include <atomic>
#include <mutex>

#include "kda_device.h"
#include "kda_host.h"

namespace {

using namespace kda;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;            // chunk length
constexpr int KD = 128;          // key width == value width
constexpr int NW = 8;            // waves per workgroup
constexpr int NT = NW * 64;      // threads per workgroup
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SCALE = 0.08838834764831845f;   // 128^-1/2
// Phase 2 block assignment, one 4-bit field per wave: blocks (3,3) (2,2)
// (1,1) (0,0) (3,2) (2,1) (1,0) (3,1).
constexpr uint32_t FULL_I = 0x31230123u;
constexpr uint32_t FULL_J = 0x10120123u;
constexpr float SAFE_EXP2 = 120.0f;             // largest split-factor exponent (base 2)
constexpr float F16_EXP2 = 14.0f;               // largest split-factor exponent for fp16 operands

// Workspace slot layout (bytes).
constexpr int WS_W = 0;
constexpr int WS_QG = WS_W + C * KD * 2;
constexpr int WS_KGT = WS_QG + C * KD * 2;
constexpr int WS_AQK = WS_KGT + KD * C * 2;
constexpr int WS_A = WS_AQK + C * C * 2;
constexpr int WS_GAM = WS_A + C * C * 2;
constexpr int WS_SLOT = WS_GAM + KD * 4;          // 66048 bytes
static_assert(WS_SLOT == KDA_PREFILL_SLOT_BYTES, "workspace slot size differs from the header's");
static_assert(WS_SLOT % 16 == 0, "slots stay 16-byte aligned");

// LDS row strides (elements).  Row strides of 68 or 36 words put eight
// consecutive rows' 16-byte accesses in distinct bank groups.  (Measured:
// the phase-2 reads, whose four lane groups sit 16 or 32 bytes apart, still
// see two-way conflicts; 288- and 544-byte strides with a channel
// permutation of G remove a third of the kernel's conflict cycles but ran no
// faster, the kernel being bound by vector ALU work and latency.)
constexpr int QS = 136;          // 16-bit [64][128] arrays
constexpr int GS = 132;          // fp32 [64][128] (G)
constexpr int LS = 68;           // fp32 [64][64] arrays
constexpr int AS = 72;           // 16-bit [*][64] arrays

// intra_kernel LDS map (bytes).  Regions are reused across phases:
//   U1   : fp32 L and T (phases 2-3), then fp16 -W (and, fused form, E^T) (phase 4)
//   AREG : fp32 scan totals (phase 1), fp16 A (phases 3-4)
constexpr int OFF_Q = 0;                                  // fp16 q^, then fp16 Qg  [64][QS]
constexpr int OFF_K = OFF_Q + C * QS * 2;                 // fp16 k^                [64][QS]
constexpr int OFF_G = OFF_K + C * QS * 2;                 // fp32 G (log2 units)    [64][GS]
constexpr int OFF_U1 = OFF_G + C * GS * 4;
constexpr int OFF_L = OFF_U1;                             // fp32 L                 [64][LS]
constexpr int OFF_T = OFF_U1 + C * LS * 4;                // fp32 (I+L)^-1          [64][LS]
constexpr int OFF_W = OFF_U1;                             // fp16 -W                [64][QS]
constexpr int OFF_ET = OFF_U1 + C * QS * 2;               // fp16 (e^G k)^T         [128][AS]
constexpr int U1_BYTES = (2 * C * LS * 4 > C * QS * 2 + KD * AS * 2) ? 2 * C * LS * 4
                                                                     : C * QS * 2 + KD * AS * 2;
constexpr int OFF_AQK = OFF_U1 + U1_BYTES;                // fp16 Aqk               [64][AS]
constexpr int OFF_A = OFF_AQK + C * AS * 2;               // fp16 A [64][AS] / scan totals
constexpr int OFF_KGT = OFF_A + C * AS * 2;               // fp16 Kg^T              [128][AS]
constexpr int OFF_BETA = OFF_KGT + KD * AS * 2;           // fp32 [64]
constexpr int OFF_GAM = OFF_BETA + C * 4;                 // fp32 [128]
constexpr int INTRA_LDS = OFF_GAM + KD * 4;
static_assert(INTRA_LDS <= 160 * 1024, "LDS budget");
// The fused form adds one v tile per wave (64 tokens x 16 columns, bf16).
constexpr int OFF_VT = INTRA_LDS;
constexpr int FUSED_LDS = OFF_VT + NW * C * 16 * 2;
static_assert(FUSED_LDS <= 160 * 1024, "LDS budget (fused)");
// The split form instead forms E^T during the solve, while U1 still holds
// T, in a region of its own past the shared map, beside the solve's Y
// blocks (which the fused form keeps in the Kg^T region).
constexpr int OFF_ETS = INTRA_LDS;                        // fp16 (e^G k)^T         [128][AS]
constexpr int OFF_YS = OFF_ETS + KD * AS * 2;             // fp32 Y20, Y21          [2][16][16]
constexpr int SPLIT_LDS = OFF_YS + 2 * 256 * 4;
static_assert(SPLIT_LDS <= 160 * 1024, "LDS budget (split)");
static_assert(C * AS * 2 >= 16 * KD * 4, "scan totals fit in the A region");
static_assert(KD * AS * 2 >= 2 * 4 * 512 * 4, "phase 2 partial sums fit in the Kg^T region");

// inter_kernel: two workgroups per (sequence, value head), each owning 64 of
// the 128 state columns with 4 waves of 16 columns.  LDS map: two verbatim
// copies of workspace slots (filled by direct global-to-LDS loads, one 1 KB
// block per wave instruction; the last block overhangs the slot, hence the
// padding) and, per wave, the v tile of its 16 columns.
constexpr int NWI = 4;                                    // waves per inter workgroup
constexpr int NTI = NWI * 64;
constexpr int VT = NWI * 16;                              // state columns per workgroup
constexpr int SLOT_U4 = WS_SLOT / 16;                     // 16-byte pieces per slot
constexpr int SLOT_BLOCKS = (WS_SLOT + 1023) / 1024;      // 1 KB load blocks per slot
constexpr int BLOCKS_PER_WAVE = (SLOT_BLOCKS + NWI - 1) / NWI;
constexpr int BUF_BYTES = SLOT_BLOCKS * 1024;
constexpr int OFF_V = 2 * BUF_BYTES;                      // bf16 [4 waves][64 tokens][CW columns]
constexpr int off_abort(int cw) { return OFF_V + NWI * C * cw * 2; }   // 4 ints: a wave gave up waiting
constexpr int inter_lds(int cw) { return off_abort(cw) + 16; }
static_assert(inter_lds(32) <= 160 * 1024, "LDS budget");
static_assert(2 * VT == KD, "two workgroups cover the state columns");

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* g;
  const uint16_t* beta;
  const float* s0;
  const int32_t* cu;
  uint16_t* o;
  float* sfin;
  unsigned char* ws;
  int64_t nslots;          // slots per value head
  int64_t w0, w1;          // slot window [w0, w1) of this launch (split form)
  int64_t wslots;          // workspace slots per value head (the window capacity)
  // Overlapped split schedule (one window): ready flags, one int per (slot,
  // value head) of the window, cleared by a small kernel before the chunk
  // kernel (intra_kernel<false, true>) sets each once its slot is stored;
  // the 32-column carry waits for them.  Null flags: sequential schedule.
  // cmajor: the chunk kernel's item i is chunk i / (N HV) of sequence
  // (i / HV) % N, value head i % HV (every sequence has T tokens), so that
  // items run in chunk rows of all units; else item i is slot i / HV of the
  // window, value head i % HV.  phase2_wgs > 0: the chunk kernel's items
  // below phase2_lo are spread over the whole grid, the rest over its first
  // phase2_wgs workgroups only, so the others leave early and the carry
  // takes their CUs.
  int* flags;
  int cmajor;
  int64_t phase2_lo;
  int phase2_wgs;
  // One word per unit after the flags, set when the unit's 32-column carry
  // gave up waiting (its slots were not stored in time, e.g. when the
  // runtime ran the carry before the chunk kernel); the sequential carry
  // launched after the join redoes exactly those units.
  int* status;
  int wait_limit;          // polls (about 55 ns each) before a carry gives up on a flag
  int T, H, HV, N;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f16x8 lds_f16x8(const uint16_t* p) {
  return *reinterpret_cast<const f16x8*>(p);
}
// Storage position of contraction index c in the "permuted" LDS layout used
// for MFMA A operands whose B operand comes straight from a float32
// accumulator: within each group of 32, index 4g + e (e < 4) goes to 8g + e
// and index 16 + 4g + e goes to 8g + 4 + e, so the 8 values lane group g
// needs for one k-step are one contiguous 16-byte read.
__device__ __forceinline__ int perm32(int c) {
  const int cp = c & 31;
  return (c & ~31) + 8 * ((cp & 15) >> 2) + 4 * (cp >> 4) + (cp & 3);
}

// Value of `v` in lane `src` (0..3) of each lane's quad.
__device__ __forceinline__ float quad_bcast(float v, int src) {
  const int x = __builtin_bit_cast(int, v);
  int r;
  switch (src) {
    case 0: r = __builtin_amdgcn_update_dpp(0, x, 0x00, 0xf, 0xf, false); break;
    case 1: r = __builtin_amdgcn_update_dpp(0, x, 0x55, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, x, 0xAA, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, x, 0xFF, 0xf, 0xf, false); break;
  }
  return __builtin_bit_cast(float, r);
}
__device__ __forceinline__ uint16_t f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  return uint32_t(f16_bits(lo)) | (uint32_t(f16_bits(hi)) << 16);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// Two bf16 values (one word) as two fp16 values (exact for the normalised
// q^, k^ entries except below 2^-14, where fp16 keeps 2^-24 absolute steps).
__device__ __forceinline__ uint32_t bf16w_to_f16w(uint32_t w) {
  const f32x2 v = {bf16lo(w), bf16hi(w)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
__device__ __forceinline__ float f16f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[0]; }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w)[1]; }

// Raw inputs of one chunk held in registers (prefetch buffer), exactly as
// loaded; rows past the chunk's end (clamped to its last row when loading)
// are zeroed only when the buffer is consumed, so that nothing touches the
// loaded registers until then and the loads stay in flight.
//   qk[2m], qk[2m+1]: q (m = 0) or k (m = 1) row tid/8, 8 bf16 at columns
//          8*(tid%8) and 64 + 8*(tid%8)
//   gv[r]: g of token 4*seg + r, channels 4*c4..4*c4+3 (seg = tid/32, c4 = tid%32)
struct Raw {
  uint4 qk[4];
  float4 gv[4];
  uint32_t beta;   // bf16 bits of beta for token tid (tid < 64)
  int nvalid;
};

// A wave-uniform global pointer, held in scalar registers.
typedef const __attribute__((address_space(1))) unsigned char* gbytes;

__device__ __forceinline__ gbytes uniform_ptr(const void* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return (gbytes)((uint64_t(hi) << 32) | lo);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_u4(gbytes base, uint32_t byte_off) {
  const u32x4_t x = *(const __attribute__((address_space(1))) u32x4_t*)(base + byte_off);
  return make_uint4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ float4 load_f4(gbytes base, uint32_t byte_off) {
  const f32x4_t x = *(const __attribute__((address_space(1))) f32x4_t*)(base + byte_off);
  return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ uint16_t load_u16(gbytes base, uint32_t byte_off) {
  return *(const __attribute__((address_space(1))) uint16_t*)(base + byte_off);
}

// q and k of the chunk: lane tid%8 of row tid/8 takes channels 8*l8..8*l8+7
// and 64+8*l8..64+8*l8+7, so each load instruction reads whole 128-byte spans.
__device__ __forceinline__ void load_raw_qk(Raw& R, const Params& p, int64_t trow, int nvalid, int hq,
                                            int tid) {
  // Scalar 64-bit bases plus 32-bit lane byte offsets.
  const int rg = tid >> 3, l8 = tid & 7;
  const uint32_t oqk = uint32_t(min(rg, nvalid - 1) * p.H * KD + 8 * l8) * 2u;
  const gbytes bq = uniform_ptr(p.q + (trow * p.H + hq) * KD);
  const gbytes bk = uniform_ptr(p.k + (trow * p.H + hq) * KD);
  R.qk[0] = load_u4(bq, oqk);
  R.qk[1] = load_u4(bq, oqk + 128u);
  R.qk[2] = load_u4(bk, oqk);
  R.qk[3] = load_u4(bk, oqk + 128u);
  R.nvalid = nvalid;
}

// g and beta of the chunk.
__device__ __forceinline__ void load_raw_g(Raw& R, const Params& p, int64_t trow, int nvalid, int hv, int tid) {
  const int seg = tid >> 5, c4 = tid & 31;
  const gbytes bg = uniform_ptr(p.g + (trow * p.HV + hv) * KD);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    R.gv[r] = load_f4(bg, uint32_t(min(4 * seg + r, nvalid - 1) * p.HV * KD + 4 * c4) * 4u);
  const gbytes bb = uniform_ptr(p.beta + trow * p.HV + hv);
  R.beta = load_u16(bb, uint32_t(min(tid & (C - 1), nvalid - 1) * p.HV) * 2u);
}

// Zero the rows of a consumed prefetch buffer that lie past the chunk's end.
// Component-wise selects: a select of whole aggregates becomes a select of
// their addresses and pushes the buffer out of registers.
__device__ __forceinline__ void mask_raw_qk(Raw& R, int tid) {
  const bool qk_ok = (tid >> 3) < R.nvalid;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    R.qk[m].x = qk_ok ? R.qk[m].x : 0u;
    R.qk[m].y = qk_ok ? R.qk[m].y : 0u;
    R.qk[m].z = qk_ok ? R.qk[m].z : 0u;
    R.qk[m].w = qk_ok ? R.qk[m].w : 0u;
  }
}

__device__ __forceinline__ void mask_raw_g(Raw& R, int tid) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const bool ok = (4 * (tid >> 5) + r) < R.nvalid;
    R.gv[r].x = ok ? R.gv[r].x : 0.f;
    R.gv[r].y = ok ? R.gv[r].y : 0.f;
    R.gv[r].z = ok ? R.gv[r].z : 0.f;
    R.gv[r].w = ok ? R.gv[r].w : 0.f;
  }
  R.beta = (tid < R.nvalid) ? R.beta : 0u;
}

// Normalise the q and k rows held in a prefetch buffer, in place.
__device__ __forceinline__ void norm_raw_qk(Raw& R, int tid) {
  mask_raw_qk(R, tid);
  l2norm_row8(R.qk[0], R.qk[1]);
  l2norm_row8(R.qk[2], R.qk[3]);
}

// cu_seqlens is read-only for the whole launch, so it is read through the
// constant address space: with a wave-uniform index the reads become scalar
// loads, which do not wait on the vector-memory counter (and so not on the
// prefetch loads in flight).
typedef const __attribute__((address_space(4))) int32_t* const_i32p;

__device__ __forceinline__ int32_t cu_at(const Params& p, int n) {
  return ((const_i32p)(p.cu))[__builtin_amdgcn_readfirstlane(n)];
}

// First token row and length of sequence n (n is wave-uniform).
__device__ __forceinline__ void seq_range(const Params& p, int n, int64_t& tok0, int& len) {
  if (p.cu) {
    const int32_t a = cu_at(p, n);
    tok0 = a;
    len = cu_at(p, n + 1) - a;
  } else {
    tok0 = int64_t(n) * p.T;
    len = p.T;
  }
}

// Workspace slot of chunk 0 of sequence n.
__device__ __forceinline__ int64_t slot_base(const Params& p, int n) {
  const int64_t tok0 = p.cu ? int64_t(cu_at(p, n)) : int64_t(n) * p.T;
  return tok0 / C + n;
}

// The sequence owning workspace slot s, or -1 for a slot between sequences.
__device__ __forceinline__ int slot_owner(const Params& p, int s, int& chunk) {
  int lo = 0, hi = p.N - 1;                 // largest n with slot_base(n) <= s
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(p, mid) <= s) lo = mid; else hi = mid - 1;
  }
  int64_t tok0;
  int len;
  seq_range(p, lo, tok0, len);
  const int64_t c = s - slot_base(p, lo);
  if (c < 0 || c * C >= len) return -1;
  chunk = int(c);
  return lo;
}

typedef __attribute__((address_space(3))) void lds_void;

constexpr int WAIT_LDS = 0xC07F;   // s_waitcnt lgkmcnt(0)
constexpr int WAIT_ALL = 0x0000;   // s_waitcnt vmcnt(0) expcnt(0) lgkmcnt(0)
// Word 3 of a raw (untyped) buffer resource on gfx9-family chips: 32-bit
// data format, no swizzle.
constexpr int BUF_RSRC_WORD3 = 0x00020000;
// Cache-policy operand of the buffer and LDS-direct memory builtins: bit 1
// nontemporal, bit 4 device scope (coherent across the XCDs' L2 caches).
constexpr int AUX_NT_DEV = 2 | 16;
constexpr int AUX_DEV = 16;
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
constexpr int WAIT_VM4 = 0x0F74;   // s_waitcnt vmcnt(4): low vmcnt bits 3:0, high bits 15:14 zero
constexpr int WAIT_VM8 = 0x0F78;   // s_waitcnt vmcnt(8)
constexpr int WAIT_VM0 = 0x0F70;   // s_waitcnt vmcnt(0) only

// Direct load of this wave's v tile (64 tokens x 16 columns from column c0,
// bf16) into its LDS region: two 1 KB blocks, lane l carrying token
// 32h + l/2, columns c0 + 8*(l&1)..+7.  Rows past the chunk's end are clamped
// here and zeroed when read.
__device__ __forceinline__ void load_v_lds(unsigned char* sv, const Params& p, int64_t trow, int nvalid,
                                           int hv, int c0, int lane) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = min(32 * h + (lane >> 1), nvalid - 1);
    const uint16_t* src = p.v + ((trow + t) * p.HV + hv) * KD + c0 + 8 * (lane & 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                     (lds_void*)(sv + h * 1024), 16, 0, 0);
  }
}

// kFused = false: the chunk-parallel half of the split form (persistent,
// items over the whole chip, outputs to the workspace).  kFused = true: the
// fused form -- one workgroup per (sequence, value head) walks its chunks in
// order and, instead of writing the chunk's matrices out, applies the carry
// to a float32 state held in registers (wave w owns state columns
// 16w..16w+15), reading every operand from LDS where phase 4 left it.
// The B operand of U = A v from a wave's v tile ([64 tokens][16 columns],
// bf16): lane (l16, gq) takes column l16 at tokens 32s + 8gq .. +7.  Each
// transposing LDS read (ds_read_b64_tr_b16) gathers, in every 16-lane group,
// element (i & 3) of the 8-byte pieces addressed by lanes (i >> 2) + 4m into
// lane i: with lane j addressing token base + (j >> 2), columns
// 4(j & 3)..+3, lane i receives column i of tokens base .. base + 3.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void read_v_operand(const unsigned char* sv, int l16, int gq, f16x8 (&Vv)[2]) {
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int base = 32 * s + 8 * gq + 4 * h;
      const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(sv + (base + (l16 >> 2)) * 32 + (l16 & 3) * 8));
#pragma unroll
      for (int m = 0; m < 4; ++m) Vv[s][4 * h + m] = (_Float16)bf16f(uint16_t(r[m]));
    }
}

// Fused form over packed sequences of different lengths: a unit's time is
// proportional to its sequence's chunk count, and workgroups start roughly in
// index order, so workgroup w takes a unit of the (w / HV)-th longest
// sequence (ties by index): longest-processing-time-first list scheduling.
// Measured on MI355X with 16 sequences of 790 to 3723 tokens x 32 value
// heads (512 units, two rounds on 256 CUs): 1.31 ms in index order, which a
// list-scheduling model at 12.5 us per chunk predicts within 1%; the model
// gives 1.00 ms longest first.  Each thread ranks one sequence against all
// others in LDS (sch: N + 1 ints of scratch), for up to NT sequences.
__device__ __forceinline__ int longest_first_seq(const Params& p, int w, int* sch, int tid) {
  const int N = p.N;
  for (int s = tid; s < N; s += NT) sch[s] = (p.cu[s + 1] - p.cu[s] + C - 1) / C;
  lds_barrier();
  if (tid < N) {
    const int mine = sch[tid];
    int rank = 0;
    for (int t = 0; t < N; ++t) {
      const int o = sch[t];
      rank += (o > mine) || (o == mine && t < tid);
    }
    if (rank == w) sch[N] = tid;   // ranks are a permutation of 0..N-1
  }
  lds_barrier();
  const int s = sch[N];
  lds_barrier();                   // the scratch is reused by the first item
  return s;
}

template <bool kFused, bool kPublish = false>
__global__ __launch_bounds__(NT) void intra_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + OFF_Q);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem + OFF_K);
  float* sG = reinterpret_cast<float*>(smem + OFF_G);
  float* sL = reinterpret_cast<float*>(smem + OFF_L);
  float* sT = reinterpret_cast<float*>(smem + OFF_T);
  uint16_t* sW = reinterpret_cast<uint16_t*>(smem + OFF_W);
  uint16_t* sET = reinterpret_cast<uint16_t*>(smem + (kFused ? OFF_ET : OFF_ETS));
  uint16_t* sAqk = reinterpret_cast<uint16_t*>(smem + OFF_AQK);
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem + OFF_A);
  float* sScr = reinterpret_cast<float*>(smem + OFF_A);
  uint16_t* sKgT = reinterpret_cast<uint16_t*>(smem + OFF_KGT);
  float* sPart = reinterpret_cast<float*>(smem + OFF_KGT);   // phase 2-3 scratch, before Kg^T
  float* sBeta = reinterpret_cast<float*>(smem + OFF_BETA);
  float* sGam = reinterpret_cast<float*>(smem + OFF_GAM);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  // Split form: work item i = slot * HV + hv; this workgroup takes items
  // blockIdx.x, blockIdx.x + gridDim.x, ...  Slots between sequences are
  // skipped.  Item ids fit in 32 bits (checked on the host).
  // Fused form: each workgroup owns one unit (sequence n, value head hv) --
  // unit w for workgroup w, or with packed sequences the longest-first order
  // above -- and its items are that sequence's chunks, in order.
  int items, stride;
  int unit_n = 0, unit_hv = 0, unit_len = 0;
  int64_t unit_tok0 = 0;
  if constexpr (kFused) {
    // The grid has exactly N * HV workgroups.
    const int w = blockIdx.x / p.HV;
    unit_hv = blockIdx.x - w * p.HV;
    unit_n = (p.cu && p.N <= NT) ? longest_first_seq(p, w, reinterpret_cast<int*>(smem + OFF_G), tid) : w;
    seq_range(p, unit_n, unit_tok0, unit_len);
    items = (unit_len + C - 1) / C;
    stride = 1;
  } else {
    items = p.cmajor ? ((p.T + C - 1) / C) * p.N * p.HV : int(p.w1 - p.w0) * p.HV;
    stride = gridDim.x;
  }
  struct Item {
    int64_t trow;
    int id, slot, hv, hq, nvalid;
  };
  // Next item id of this workgroup.  Overlapped schedule: items below
  // phase2_lo over the whole grid, the rest over its first phase2_wgs
  // workgroups (w2 >= 0, their order there); the others leave.  Below
  // phase2_lo the first (phase2_lo mod grid) workgroups take one item more;
  // the order is rotated so that the next ones take the rest's short last
  // round, and the workgroups that stay end within one item of each other.
  int w2 = -1;
  if (!kFused && int(blockIdx.x) < p.phase2_wgs) {
    const int extra1 = int(p.phase2_lo % int64_t(gridDim.x)) % p.phase2_wgs;
    w2 = (int(blockIdx.x) + p.phase2_wgs - extra1) % p.phase2_wgs;
  }
  auto next_of = [&](int id) __attribute__((always_inline)) {
    if (kFused || p.phase2_wgs == 0) return id + stride;
    const int p1 = int(p.phase2_lo);
    if (id < p1) {
      const int n = id + stride;
      if (n < p1) return n;
      return w2 >= 0 ? p1 + w2 : items;
    }
    return id + p.phase2_wgs;
  };
  auto find = [&](int i) {
    Item it;
    if constexpr (kFused) {
      it.id = i;
      it.trow = unit_tok0 + int64_t(i) * C;
      it.nvalid = min(C, unit_len - i * C);
      it.slot = i;
      it.hv = unit_hv;
      it.hq = unit_hv / (p.HV / p.H);
      return it;
    }
    if (p.cmajor) {
      if (i < items) {
        const int units = p.N * p.HV;
        const int c = i / units;
        const int n = (i - c * units) / p.HV;
        it.hv = i - c * units - n * p.HV;
        it.trow = int64_t(n) * p.T + int64_t(c) * C;
        it.nvalid = min(C, p.T - c * C);
        it.slot = int(slot_base(p, n)) + c;
        it.hq = it.hv / (p.HV / p.H);
      }
      it.id = i;
      return it;
    }
    for (; i < items; i = next_of(i)) {
      const int s = int(p.w0) + i / p.HV;
      int c;
      const int n = slot_owner(p, s, c);
      if (n < 0) continue;
      int64_t tok0;
      int len;
      seq_range(p, n, tok0, len);
      it.trow = tok0 + int64_t(c) * C;
      it.nvalid = min(C, len - c * C);
      it.slot = s;
      it.hv = i - (s - int(p.w0)) * p.HV;
      it.hq = it.hv / (p.HV / p.H);
      break;
    }
    it.id = i;
    return it;
  };

  // Fused form: this wave's 128x16 slice of the state (rows 16rt + 4gq + r of
  // column 16 * wave + l16), float32, for the whole sequence.
  f32x4 S[8];
  unsigned char* sVt = smem + OFF_VT + wave * (C * 16 * 2);
  if constexpr (kFused) {
    const int col = 16 * wave + l16;
    if (p.s0) {   // one branch around all 32 loads, so they are in flight together
      const float* s0 = p.s0 + (int64_t(unit_n) * p.HV + unit_hv) * KD * KD;
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[rt][r] = s0[(16 * rt + 4 * gq + r) * KD + col];
    } else {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  auto write_final_state = [&]() __attribute__((always_inline)) {
    if constexpr (kFused) {
      float* sf = p.sfin + (int64_t(unit_n) * p.HV + unit_hv) * KD * KD;
      const int col = 16 * wave + l16;
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sf[(16 * rt + 4 * gq + r) * KD + col] = S[rt][r];
    }
  };

  // E^T = (e^G k)^T and Kg^T = (k e^{G_last - G})^T into LDS, and Qg of this
  // thread's entries into `qg` (stored by store_qg once no thread reads q^
  // any more).  Thread t handles channels c2, c2+1 (c2 = 2*(t%64)) for
  // tokens 8*(t/64)..+7.
  auto form_egk = [&](uint32_t (&qg_pk)[8]) __attribute__((always_inline)) {
    const int c2 = 2 * (tid & 63);
    const int j0 = 8 * (tid >> 6);
    const float2 glast = *reinterpret_cast<const float2*>(sG + (C - 1) * GS + c2);
    float ev0[8], ev1[8], kv0[8], kv1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int jj = j0 + e;
      const float2 gj = *reinterpret_cast<const float2*>(sG + jj * GS + c2);
      const uint32_t kk = *reinterpret_cast<const uint32_t*>(sK + jj * QS + c2);
      const uint32_t qq = *reinterpret_cast<const uint32_t*>(sQ + jj * QS + c2);
      const float eg0 = ex2(gj.x), eg1 = ex2(gj.y);
      const float k0 = f16lo(kk), k1 = f16hi(kk);
      ev0[e] = k0 * eg0;
      ev1[e] = k1 * eg1;
      kv0[e] = k0 * ex2(glast.x - gj.x);
      kv1[e] = k1 * ex2(glast.y - gj.y);
      qg_pk[e] = pack_f16(SCALE * f16lo(qq) * eg0, SCALE * f16hi(qq) * eg1);
    }
    *reinterpret_cast<uint4*>(sET + c2 * AS + j0) =
        make_uint4(pack_f16(ev0[0], ev0[1]), pack_f16(ev0[2], ev0[3]), pack_f16(ev0[4], ev0[5]), pack_f16(ev0[6], ev0[7]));
    *reinterpret_cast<uint4*>(sET + (c2 + 1) * AS + j0) =
        make_uint4(pack_f16(ev1[0], ev1[1]), pack_f16(ev1[2], ev1[3]), pack_f16(ev1[4], ev1[5]), pack_f16(ev1[6], ev1[7]));
    // Kg^T in the permuted token layout: tokens j0..j0+3 and j0+4..j0+7 each
    // land as one contiguous 8-byte group.
    const int pj0 = perm32(j0), pj4 = perm32(j0 + 4);
    *reinterpret_cast<uint2*>(sKgT + c2 * AS + pj0) = make_uint2(pack_f16(kv0[0], kv0[1]), pack_f16(kv0[2], kv0[3]));
    *reinterpret_cast<uint2*>(sKgT + c2 * AS + pj4) = make_uint2(pack_f16(kv0[4], kv0[5]), pack_f16(kv0[6], kv0[7]));
    *reinterpret_cast<uint2*>(sKgT + (c2 + 1) * AS + pj0) = make_uint2(pack_f16(kv1[0], kv1[1]), pack_f16(kv1[2], kv1[3]));
    *reinterpret_cast<uint2*>(sKgT + (c2 + 1) * AS + pj4) = make_uint2(pack_f16(kv1[4], kv1[5]), pack_f16(kv1[6], kv1[7]));
  };
  // Qg over q^ in the permuted channel layout; c2 and c2 + 1 stay adjacent
  // there.
  auto store_qg = [&](const uint32_t (&qg_pk)[8]) __attribute__((always_inline)) {
    const int pc = perm32(2 * (tid & 63));
    const int j0 = 8 * (tid >> 6);
#pragma unroll
    for (int e = 0; e < 8; ++e) *reinterpret_cast<uint32_t*>(sQ + (j0 + e) * QS + pc) = qg_pk[e];
  };

  // Overlapped schedule: the flag index (slot, value head) of the item whose
  // slot stores are in flight, and the release of its flag (a device-scope
  // store, which the carry polls).
  int pend = -1;
  auto publish = [&](int id) __attribute__((always_inline)) {
    __hip_atomic_store(p.flags + id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int first_id = kFused ? 0 : int(blockIdx.x);
  if (!kFused && p.phase2_wgs > 0 && first_id >= int(p.phase2_lo))
    first_id = w2 >= 0 ? int(p.phase2_lo) + w2 : items;
  Item first = find(first_id);
  if (first.id >= items) {
    write_final_state();   // fused form, empty sequence: the state passes through
    return;
  }
  Raw R;
  load_raw_qk(R, p, first.trow, first.nvalid, first.hq, tid);
  load_raw_g(R, p, first.trow, first.nvalid, first.hv, tid);

  // Fused form: the carry of chunk `cur` on this wave's 16 state columns,
  //   U = A v,  Vnew = U - W S,  O = Qg S + Aqk Vnew,
  //   S = e^{G_last} S + Kg^T Vnew,
  // on MFMA with the operands where phase 4 left them in LDS (logical
  // order; W, Qg, Kg^T and Aqk in the permuted contraction order that lets
  // the float32 accumulators serve directly as fp16 operands).
  auto carry = [&](const Item& cur) __attribute__((always_inline)) {
    const int c0 = 16 * wave;
    // The v tile was loaded with direct global-to-LDS loads by this wave.
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    f16x8 Vv[2];
    read_v_operand(sVt, l16, gq, Vv);
    f16x8 Sh[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Sh[s][r] = (_Float16)S[2 * s][r];
        Sh[s][4 + r] = (_Float16)S[2 * s + 1][r];
      }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
      const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 16 * rt + 4 * gq);
#pragma unroll
      for (int r = 0; r < 4; ++r) S[rt][r] *= gm[r];
    }
    // U = A v, then Vnew = U + (-W) S; A is lower triangular.
    f32x4 Vn[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq), Vv[s],
                                                     acc, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16x8(sW + (16 * mt + l16) * QS + 32 * s + 8 * gq), Sh[s],
                                                     acc, 0, 0, 0);
      Vn[mt] = acc;
    }
    f16x8 Vh[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Vh[s][r] = (_Float16)Vn[2 * s][r];
        Vh[s][4 + r] = (_Float16)Vn[2 * s + 1][r];
      }
    // O^T = S^T Qg^T + Vnew^T Aqk^T: each lane ends with four adjacent
    // columns of one token.
    const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
        p.o + (cur.trow * p.HV + cur.hv) * KD, 0, cur.nvalid * p.HV * KD * 2, BUF_RSRC_WORD3);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sh[s], lds_f16x8(sQ + (16 * mt + l16) * QS + 32 * s + 8 * gq),
                                                     acc, 0, 0, 0);
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vh[s], lds_f16x8(sAqk + (16 * mt + l16) * AS + 32 * s + 8 * gq),
                                                     acc, 0, 0, 0);
      const int t = 16 * mt + l16;
      const u32x2_t w = {pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
      __builtin_amdgcn_raw_buffer_store_b64(w, orsrc, (t * p.HV * KD + c0 + 4 * gq) * 2, 0, 0);
    }
    // S = (e^{G_last} S) + Kg^T Vnew.
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        S[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(lds_f16x8(sKgT + (16 * rt + l16) * AS + 32 * s + 8 * gq), Vh[s],
                                                       S[rt], 0, 0, 0);
  };

  // One chunk item: consumes R (cur's inputs), refills it with nxt's.
  // `first`: q and k of this item were not normalised at the end of the
  // previous one.
  auto chunk = [&](const Item& cur, const Item& nxt, const bool first) __attribute__((always_inline)) {
    const int hv = cur.hv;
    (void)hv;

    // ---------------------------------------------------------- phase 1
    {
      // q^ and k^: one 8-lane group per row, bit-exact normalisation (done at
      // the end of the previous item, except for a workgroup's first).
      if (first) norm_raw_qk(R, tid);
      mask_raw_g(R, tid);
      {
        const int rg = tid >> 3, l8 = tid & 7;
        // Staged as fp16, the MFMA operand type (see the precision note at
        // the top of this file).
        uint4 h[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          h[m] = make_uint4(bf16w_to_f16w(R.qk[m].x), bf16w_to_f16w(R.qk[m].y), bf16w_to_f16w(R.qk[m].z),
                            bf16w_to_f16w(R.qk[m].w));
        *reinterpret_cast<uint4*>(sQ + rg * QS + 8 * l8) = h[0];
        *reinterpret_cast<uint4*>(sQ + rg * QS + 64 + 8 * l8) = h[1];
        *reinterpret_cast<uint4*>(sK + rg * QS + 8 * l8) = h[2];
        *reinterpret_cast<uint4*>(sK + rg * QS + 64 + 8 * l8) = h[3];
      }
      if (tid < C) sBeta[tid] = bf16f(uint16_t(R.beta));
      // g in log2 units, inclusive scan over the 4 tokens this thread holds,
      // then across the 16 four-token segments through LDS.
      const int seg = tid >> 5, c4 = tid & 31;
      float4 gs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gs[r].x = R.gv[r].x * LOG2E + (r ? gs[r - 1].x : 0.f);
        gs[r].y = R.gv[r].y * LOG2E + (r ? gs[r - 1].y : 0.f);
        gs[r].z = R.gv[r].z * LOG2E + (r ? gs[r - 1].z : 0.f);
        gs[r].w = R.gv[r].w * LOG2E + (r ? gs[r - 1].w : 0.f);
      }
      *reinterpret_cast<float4*>(sScr + seg * KD + 4 * c4) = gs[3];
      lds_barrier();
      // Exclusive prefix of the 16 segment totals, one thread per channel,
      // written back in place.
      if (tid < KD) {
        float t[16];
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) t[s2] = sScr[s2 * KD + tid];
        float run = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
          sScr[s2 * KD + tid] = run;
          run += t[s2];
        }
      }
      lds_barrier();
      const float4 off = *reinterpret_cast<const float4*>(sScr + seg * KD + 4 * c4);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(sG + (4 * seg + r) * GS + 4 * c4) =
            make_float4(gs[r].x + off.x, gs[r].y + off.y, gs[r].z + off.z, gs[r].w + off.w);
    }
    lds_barrier();

    // ---------------------------------------------------------- phase 2: L, Aqk
    // The raw registers are consumed: prefetch the next chunk, q and k now,
    // g and beta at the start of phase 3, so that the loads do not all queue
    // in the memory pipe at once.
    if (nxt.id < items) load_raw_qk(R, p, nxt.trow, nxt.nvalid, nxt.hq, tid);
    // The 10 blocks on or below the diagonal: wave w computes one whole block
    // (FULL_I/J below) plus one 32-channel quarter of one of the two blocks
    // (3,0) and (2,0), whose four partial products are summed after the
    // barrier.  Waves 2..7 also zero one strictly-upper block of Aqk each.
    {
      if (wave >= 2) {
        const int ub = wave - 2;
        const int UI = ub < 3 ? 0 : (ub < 5 ? 1 : 2);
        const int UJ = ub < 3 ? ub + 1 : (ub < 5 ? ub - 1 : 3);
#pragma unroll
        for (int r = 0; r < 4; ++r) sAqk[(16 * UI + 4 * gq + r) * AS + perm32(16 * UJ + l16)] = 0;
      }
      {
        const int I = (FULL_I >> (4 * wave)) & 15;
        const int J = (FULL_J >> (4 * wave)) & 15;
        const int ref = (J < I) ? 16 * I : 16 * I + 8;
        const int i = 16 * I + l16;     // operand row (A side)
        const int j = 16 * J + l16;     // operand row (B side)
        // Largest split-factor exponent of this lane's entries (<= 0 below the
        // diagonal, so only diagonal blocks need the check).  In the split
        // form a diagonal block forms all four k-steps' factors and fp16
        // operands first, taking the exponents' largest magnitude on the way
        // (on a diagonal block j == i, so the two factors' exponents are
        // G_i - G_ref and its negation), and runs the products once the range
        // is known.
        float emax = 0.f;
        f32x4 accL = {0.f, 0.f, 0.f, 0.f};
        f32x4 accQ = {0.f, 0.f, 0.f, 0.f};
        auto factors = [&](int s, f32x8& fr, f32x8& fc, float* em) __attribute__((always_inline)) {
          const int ch0 = 32 * s + 8 * gq;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const float4 gi4 = *reinterpret_cast<const float4*>(sG + i * GS + ch0 + 4 * h);
            const float4 gj4 = *reinterpret_cast<const float4*>(sG + j * GS + ch0 + 4 * h);
            const float4 gr4 = *reinterpret_cast<const float4*>(sG + ref * GS + ch0 + 4 * h);
            const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
            const float gj[4] = {gj4.x, gj4.y, gj4.z, gj4.w};
            const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float d = gi[e] - gr[e];
              if (em) *em = fmaxf(*em, fabsf(d));
              fr[4 * h + e] = ex2(d);
              fc[4 * h + e] = ex2(gr[e] - gj[e]);
            }
          }
        };
        bool wide = false;
        if constexpr (kFused) {
          // (The fused form, whose carry state holds more registers, keeps a
          // separate pass over the exponents: folded in, it spills.)
          if (J == I) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int ch0 = 32 * s + 8 * gq;
#pragma unroll
              for (int h = 0; h < 2; ++h) {
                const float4 gi = *reinterpret_cast<const float4*>(sG + i * GS + ch0 + 4 * h);
                const float4 gr = *reinterpret_cast<const float4*>(sG + ref * GS + ch0 + 4 * h);
                emax = fmaxf(emax, fmaxf(fmaxf(fabsf(gi.x - gr.x), fabsf(gi.y - gr.y)),
                                         fmaxf(fabsf(gi.z - gr.z), fabsf(gi.w - gr.w))));
              }
            }
          }
          wide = __any(emax > F16_EXP2);
        }
        if (!kFused && J == I) {
          f16x8 aL[4], aQ[4], bK[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int ch0 = 32 * s + 8 * gq;
            const f16x8 ki = *reinterpret_cast<const f16x8*>(sK + i * QS + ch0);
            const f16x8 qi = *reinterpret_cast<const f16x8*>(sQ + i * QS + ch0);
            const f16x8 kj = *reinterpret_cast<const f16x8*>(sK + j * QS + ch0);
            f32x8 fr, fc;
            factors(s, fr, fc, &emax);
            const f16x8 frh = __builtin_convertvector(fr, f16x8);
            const f16x8 fch = __builtin_convertvector(fc, f16x8);
            aL[s] = ki * frh;
            aQ[s] = qi * frh;
            bK[s] = kj * fch;
          }
          wide = __any(emax > F16_EXP2);
          if (!wide) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(aL[s], bK[s], accL, 0, 0, 0);
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(aQ[s], bK[s], accQ, 0, 0, 0);
            }
          }
        }
        if (kFused || J != I || wide) {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int ch0 = 32 * s + 8 * gq;
            const f16x8 ki = *reinterpret_cast<const f16x8*>(sK + i * QS + ch0);
            const f16x8 qi = *reinterpret_cast<const f16x8*>(sQ + i * QS + ch0);
            const f16x8 kj = *reinterpret_cast<const f16x8*>(sK + j * QS + ch0);
            f32x8 fr, fc;
            factors(s, fr, fc, nullptr);
            if (!wide) {
              // Split factors rounded to fp16, products in packed fp16.
              const f16x8 frh = __builtin_convertvector(fr, f16x8);
              const f16x8 fch = __builtin_convertvector(fc, f16x8);
              accL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ki * frh, kj * fch, accL, 0, 0, 0);
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(qi * frh, kj * fch, accQ, 0, 0, 0);
            } else {
              // Steep decay inside a diagonal block: bf16 operands keep the range.
              bf16x8 a, b, c;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                a[e] = (__bf16)((float)ki[e] * fr[e]);
                b[e] = (__bf16)((float)qi[e] * fr[e]);
                c[e] = (__bf16)((float)kj[e] * fc[e]);
              }
              accL = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, c, accL, 0, 0, 0);
              accQ = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, c, accQ, 0, 0, 0);
            }
          }
        }
        const int jc = 16 * J + l16;    // result column
        if (__any(emax > SAFE_EXP2)) {
          // Extreme decay inside a diagonal block: evaluate each pair directly.
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ir = 16 * I + 4 * gq + r;
            float aL = 0.f, aQ = 0.f;
            if (jc <= ir) {
              for (int ch = 0; ch < KD; ++ch) {
                const float f = ex2(sG[ir * GS + ch] - sG[jc * GS + ch]);
                const float kjf = f16f(sK[jc * QS + ch]) * f;
                aL = fmaf(f16f(sK[ir * QS + ch]), kjf, aL);
                aQ = fmaf(f16f(sQ[ir * QS + ch]), kjf, aQ);
              }
            }
            accL[r] = aL;
            accQ[r] = aQ;
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int ir = 16 * I + 4 * gq + r;
          sL[ir * LS + jc] = (jc < ir) ? sBeta[ir] * accL[r] : 0.f;
          sAqk[ir * AS + perm32(jc)] = f16_bits((jc <= ir) ? SCALE * accQ[r] : 0.f);
        }
      }
      {
        // Quarter (channels 32s..32s+31) of block (I, 0), I = 3 - wave/4:
        // below the diagonal, so both split factors are <= 1.
        const int X = wave >> 2;
        const int I = 3 - X;
        const int s = wave & 3;
        const int i = 16 * I + l16;
        const int j = l16;
        const int ch0 = 32 * s + 8 * gq;
        const f16x8 ki = *reinterpret_cast<const f16x8*>(sK + i * QS + ch0);
        const f16x8 qi = *reinterpret_cast<const f16x8*>(sQ + i * QS + ch0);
        const f16x8 kj = *reinterpret_cast<const f16x8*>(sK + j * QS + ch0);
        f32x8 fr, fc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float4 gi4 = *reinterpret_cast<const float4*>(sG + i * GS + ch0 + 4 * h);
          const float4 gj4 = *reinterpret_cast<const float4*>(sG + j * GS + ch0 + 4 * h);
          const float4 gr4 = *reinterpret_cast<const float4*>(sG + 16 * I * GS + ch0 + 4 * h);
          const float gi[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
          const float gj[4] = {gj4.x, gj4.y, gj4.z, gj4.w};
          const float gr[4] = {gr4.x, gr4.y, gr4.z, gr4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            fr[4 * h + e] = ex2(gi[e] - gr[e]);
            fc[4 * h + e] = ex2(gr[e] - gj[e]);
          }
        }
        const f16x8 frh = __builtin_convertvector(fr, f16x8);
        const f16x8 fch = __builtin_convertvector(fc, f16x8);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 pL = __builtin_amdgcn_mfma_f32_16x16x32_f16(ki * frh, kj * fch, z, 0, 0, 0);
        const f32x4 pQ = __builtin_amdgcn_mfma_f32_16x16x32_f16(qi * frh, kj * fch, z, 0, 0, 0);
        float* part = sPart + (X * 4 + s) * 512;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          part[(4 * gq + r) * 16 + l16] = pL[r];
          part[256 + (4 * gq + r) * 16 + l16] = pQ[r];
        }
      }
    }
    // Overlapped schedule: the previous item's 9 slot stores precede this
    // item's 4 q/k prefetch loads (none after the last item) in the in-order
    // completion counter, so this wait completes exactly those stores (issued
    // an item's first two phases ago); their flag is set after the barrier
    // below, once every thread has waited.
    if constexpr (kPublish) {
      if (pend >= 0) {
        if (nxt.id < items) __builtin_amdgcn_s_waitcnt(WAIT_VM4);
        else __builtin_amdgcn_s_waitcnt(WAIT_VM0);
      }
    }
    lds_barrier();
    if constexpr (kPublish) {
      if (pend >= 0 && tid == 0) publish(pend);
    }

    // ---------------------------------------------------------- phase 3: solve
    if (nxt.id < items) load_raw_g(R, p, nxt.trow, nxt.nvalid, nxt.hv, tid);
    // Fused form: this chunk's v tile for the wave's 16 state columns, for
    // the carry at the end of the item.
    if constexpr (kFused) load_v_lds(sVt, p, cur.trow, cur.nvalid, cur.hv, 16 * wave, lane);
    // T = (I + L)^-1, unit lower triangular.
    // Diagonal 16x16 blocks: wave b < 4 inverts block b.  Lane 4*cc + h holds
    // rows 4h..4h+3 of column cc and the matching rows of L in registers;
    // column-oriented forward substitution broadcasts x[m] within the quad.
    if (wave < 4) {
      const int blk = wave;
      const int cc = lane >> 2;
      const int h = lane & 3;
      float Lr[4][16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ii = 4 * h + r;
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
          const float4 l4 = *reinterpret_cast<const float4*>(sL + (16 * blk + ii) * LS + 16 * blk + 4 * m4);
          Lr[r][4 * m4 + 0] = (4 * m4 + 0 < ii) ? l4.x : 0.f;
          Lr[r][4 * m4 + 1] = (4 * m4 + 1 < ii) ? l4.y : 0.f;
          Lr[r][4 * m4 + 2] = (4 * m4 + 2 < ii) ? l4.z : 0.f;
          Lr[r][4 * m4 + 3] = (4 * m4 + 3 < ii) ? l4.w : 0.f;
        }
      }
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = (4 * h + r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < 15; ++m) {
        // x[m] lives in quad lane m/4, register m%4; broadcast it to the quad.
        const float xm = quad_bcast(x[m & 3], m >> 2);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = fmaf(-Lr[r][m], xm, x[r]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) sT[(16 * blk + 4 * h + r) * LS + 16 * blk + cc] = x[r];
    } else {
      // Meanwhile waves 4..7 finish blocks (3,0) and (2,0) of L and Aqk: the
      // four quarter products are summed in channel order.
      // Wave 4 + k takes block X = k / 2, matrix k % 2 (L or Aqk); lane l
      // sums entries 4l..4l+3 (row l / 4, columns 4 (l % 4)..+3).
      const int k = wave - 4;
      const int X = k >> 1;
      const float* part = sPart + X * 4 * 512 + (k & 1) * 256 + 4 * lane;
      const float4 p0 = *reinterpret_cast<const float4*>(part);
      const float4 p1 = *reinterpret_cast<const float4*>(part + 512);
      const float4 p2 = *reinterpret_cast<const float4*>(part + 1024);
      const float4 p3 = *reinterpret_cast<const float4*>(part + 1536);
      const float v[4] = {((p0.x + p1.x) + p2.x) + p3.x, ((p0.y + p1.y) + p2.y) + p3.y,
                          ((p0.z + p1.z) + p2.z) + p3.z, ((p0.w + p1.w) + p2.w) + p3.w};
      const int ir = 16 * (3 - X) + (lane >> 2), jc = 4 * (lane & 3);
      if ((k & 1) == 0) {
        const float bi = sBeta[ir];
        *reinterpret_cast<float4*>(sL + ir * LS + jc) = make_float4(bi * v[0], bi * v[1], bi * v[2], bi * v[3]);
      } else {
        *reinterpret_cast<uint2*>(sAqk + ir * AS + perm32(jc)) =
            make_uint2(pack_f16(SCALE * v[0], SCALE * v[1]), pack_f16(SCALE * v[2], SCALE * v[3]));
      }
    }
    lds_barrier();
    // Split form: E^T (in its own region), Kg^T (in its region, whose phase-2
    // partial sums were consumed above) and Qg (in registers) are formed
    // here, so that their vector work runs beside the MFMA chains of the
    // off-diagonal steps below; Qg is stored over q^ after the first step's
    // barrier, when no thread reads q^ any more.
    uint32_t qg_pk[8];
    if constexpr (!kFused) form_egk(qg_pk);
    // Off-diagonal blocks of T on fp32 MFMA (16x16x4), through the inverse
    // of the two 32x32 diagonal halves Z0 = [[T00, 0], [T10, T11]] and
    // Z1 = [[T22, 0], [T32, T33]]:
    //   T10 = -T11 L10 T00,  T32 = -T33 L32 T22,
    //   [[T20, T21], [T30, T31]] = -Z1 Y,  Y = [[L20, L21], [L30, L31]] Z0,
    // in three steps whose longest dependent chain is 8 + 4 + 8 MFMAs.
    // In k-step s, lane group gq takes contraction index 4gq + s for
    // products whose right operand is an accumulator (which holds exactly
    // those entries) and 4s + gq when both operands come from LDS.
    {
      // Y20 and Y21, 16x16 row-major (fused form: where the partial sums,
      // consumed above, were).
      float* sY20 = kFused ? sPart : reinterpret_cast<float*>(smem + OFF_YS);
      float* sY21 = sY20 + 256;
      // acc += L_IM T_MJ, both from LDS.
      auto lt = [&](f32x4 acc, int I, int M, int J) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sL[(16 * I + l16) * LS + 16 * M + 4 * s + gq],
                                                     sT[(16 * M + 4 * s + gq) * LS + 16 * J + l16], acc, 0, 0, 0);
        return acc;
      };
      // acc -= T_IK P, P an accumulator.
      auto tp = [&](f32x4 acc, int I, int K, const f32x4& P) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-sT[(16 * I + l16) * LS + 16 * K + 4 * gq + s], P[s], acc, 0, 0, 0);
        return acc;
      };
      // acc -= T_IK Y, Y a 16x16 block in LDS.
      auto ty = [&](f32x4 acc, int I, int K, const float* Y) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-sT[(16 * I + l16) * LS + 16 * K + 4 * s + gq],
                                                     Y[(4 * s + gq) * 16 + l16], acc, 0, 0, 0);
        return acc;
      };
      auto put_t = [&](const f32x4& X, int I, int J) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sT[(16 * I + 4 * gq + r) * LS + 16 * J + l16] = X[r];
      };
      auto put_y = [&](const f32x4& X, float* Y) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[(4 * gq + r) * 16 + l16] = X[r];
      };
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 Y = z;
      // Step 1: T10, T32; Y21, Y31 and the T00 terms of Y20, Y30.
      if (wave == 0) put_t(tp(z, 1, 1, lt(z, 1, 0, 0)), 1, 0);
      else if (wave == 1) put_t(tp(z, 3, 3, lt(z, 3, 2, 2)), 3, 2);
      else if (wave == 2) { Y = lt(z, 2, 1, 1); put_y(Y, sY21); }
      else if (wave == 3) Y = lt(z, 3, 1, 1);
      else if (wave == 4) Y = lt(z, 2, 0, 0);
      else if (wave == 5) Y = lt(z, 3, 0, 0);
      lds_barrier();
      if constexpr (!kFused) store_qg(qg_pk);
      // Step 2: the T10 terms of Y20, Y30.
      if (wave == 4) { Y = lt(Y, 2, 1, 0); put_y(Y, sY20); }
      else if (wave == 5) Y = lt(Y, 3, 1, 0);
      lds_barrier();
      // Step 3: T20, T21, T30, T31.
      if (wave == 4) put_t(tp(z, 2, 2, Y), 2, 0);
      else if (wave == 2) put_t(tp(z, 2, 2, Y), 2, 1);
      else if (wave == 5) put_t(tp(ty(z, 3, 2, sY20), 3, 3, Y), 3, 0);
      else if (wave == 3) put_t(tp(ty(z, 3, 2, sY21), 3, 3, Y), 3, 1);
      lds_barrier();
    }
    // A = T diag(beta), lower triangular, as fp16 (8 entries per thread).
    {
      const int ii = tid >> 3;
      const int j0 = 8 * (tid & 7);
      const float4 t0 = *reinterpret_cast<const float4*>(sT + ii * LS + j0);
      const float4 t1 = *reinterpret_cast<const float4*>(sT + ii * LS + j0 + 4);
      const float4 b0 = *reinterpret_cast<const float4*>(sBeta + j0);
      const float4 b1 = *reinterpret_cast<const float4*>(sBeta + j0 + 4);
      const float tv[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
      const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = (j0 + e <= ii) ? tv[e] * bv[e] : 0.f;
      *reinterpret_cast<uint4*>(sA + ii * AS + j0) =
          make_uint4(pack_f16(a[0], a[1]), pack_f16(a[2], a[3]), pack_f16(a[4], a[5]), pack_f16(a[6], a[7]));
    }
    if (tid < KD) sGam[tid] = ex2(sG[(C - 1) * GS + tid]);
    lds_barrier();

    // ---------------------------------------------------------- phase 4: E, Kg, Qg, W
    // (Split form: E^T, Kg^T and Qg were formed during the solve.)
    if constexpr (kFused) {
      uint32_t qg_fused[8];
      form_egk(qg_fused);
      lds_barrier();
      store_qg(qg_fused);
    }
    // W = A (e^G k): 4 x 8 output tiles, 4 per wave; A is lower triangular.
    // Computed as W^T = E^T A^T (the same two operand reads, roles swapped),
    // so each lane holds four adjacent channels of one token; -W is stored in
    // the permuted channel layout, where those four stay adjacent (8 bytes).
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int pt = wave + NW * q4;
      const int mt = pt >> 3;
      const int nt = pt & 7;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s <= (mt >> 1); ++s) {
        const f16x8 a = lds_f16x8(sA + (16 * mt + l16) * AS + 32 * s + 8 * gq);
        const f16x8 b = lds_f16x8(sET + (16 * nt + l16) * AS + 32 * s + 8 * gq);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, acc, 0, 0, 0);
      }
      *reinterpret_cast<uint2*>(sW + (16 * mt + l16) * QS + perm32(16 * nt + 4 * gq)) =
          make_uint2(pack_f16(-acc[0], -acc[1]), pack_f16(-acc[2], -acc[3]));
    }
    lds_barrier();

    if constexpr (!kFused) {
    // Chunk outputs -> workspace slot, in slot order (coalesced 16-byte
    // stores), gathering each piece from its swizzled source position.  A
    // fixed number of unconditional stores per thread (the overhang repeats
    // the slot's last piece) keeps the store count known at compile time, so
    // the next chunk waits only for its prefetched inputs, not for these.
    // The stores carry the nontemporal hint (the slot is read back once, by
    // the other kernel, long after it has left the caches), measured ~1%
    // faster; the same hint on the input loads or on the other kernel's
    // slot, v and o traffic measured slower.
    {
      unsigned char* dst = p.ws + (int64_t(cur.hv) * p.wslots + (cur.slot - p.w0)) * WS_SLOT;
      // kPublish: device-scope stores, since the carry reads the slot while
      // this kernel runs, maybe from another XCD, once its stores are
      // complete (kernel boundaries publish the other launches' slots).
      const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(dst, 0, WS_SLOT, BUF_RSRC_WORD3);
#pragma unroll
      for (int k = 0; k < (SLOT_U4 + NT - 1) / NT; ++k) {
        const int u = min(tid + k * NT, SLOT_U4 - 1);
        const int b = u * 16;
        const unsigned char* src;
        if (b < WS_KGT) {          // W, Qg: 64 rows of 16 pieces
          const int off = b < WS_QG ? b : b - WS_QG;
          const int r = off >> 8, pp = (off >> 4) & 15;
          const uint16_t* base = b < WS_QG ? sW : sQ;
          src = reinterpret_cast<const unsigned char*>(base + r * QS) + ((pp ^ (r & 7)) << 4);
        } else if (b < WS_GAM) {   // Kg^T, Aqk, A: rows of 8 pieces
          const uint16_t* base;
          int off;
          if (b < WS_AQK) { base = sKgT; off = b - WS_KGT; }
          else if (b < WS_A) { base = sAqk; off = b - WS_AQK; }
          else { base = sA; off = b - WS_A; }
          const int r = off >> 7, pp = (off >> 4) & 7;
          src = reinterpret_cast<const unsigned char*>(base + r * AS) + ((pp ^ (r & 7)) << 4);
        } else {
          src = reinterpret_cast<const unsigned char*>(sGam) + (b - WS_GAM);
        }
        const uint4 val = *reinterpret_cast<const uint4*>(src);
        if constexpr (kPublish) {
          const u32x4_t w = {val.x, val.y, val.z, val.w};
          __builtin_amdgcn_raw_buffer_store_b128(w, srsrc, b, 0, AUX_NT_DEV);
        } else {
          kda::store_nt(reinterpret_cast<uint4*>(dst + b), val);
        }
      }
      pend = (cur.slot - int(p.w0)) * p.HV + cur.hv;
    }
    } else {
      carry(cur);
    }
    // While those stores drain (the vector ALUs are otherwise idle here),
    // normalise the next item's q and k, prefetched in phase 2.  (Fused
    // form: after the carry.)
    if (nxt.id < items) norm_raw_qk(R, tid);
    lds_barrier();
  };

  // Loads and stores share one in-order completion counter.  Every item
  // issues the next item's loads and then its own 9 workspace stores, so the
  // wait for the prefetched registers may leave those stores in flight.  The
  // first item is peeled off the loop so that the loop is entered in that
  // same state; with a plain loop the entry path (loads only) would make the
  // compiler's wait at the loop head conservative and drain the stores too.
  Item nxt = find(next_of(first.id));
  chunk(first, nxt, true);
  while (nxt.id < items) {
    const Item cur = nxt;
    nxt = find(next_of(cur.id));
    chunk(cur, nxt, false);
  }
  if constexpr (kPublish) {   // the last item's flag, once its stores are complete
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
    lds_barrier();
    if (tid == 0) publish(pend);
  }
  write_final_state();
}

// Direct global-to-LDS copy of part of one workspace slot: 1 KB blocks,
// wave w issuing blocks w, w + 4, ... (its j-th block for j in [j0, j1)).
// Each lane moves 16 bytes to the block base + 16 * lane; pieces past the end
// of the slot re-read its last piece into the buffer's padding, and a wave
// with fewer blocks repeats the last block (same bytes to the same place), so
// every wave issues the same number of loads.
template <int AUX = 0>
__device__ __forceinline__ void load_slot_part(unsigned char* buf, const unsigned char* slot, int wave, int lane,
                                               int j0, int j1) {
#pragma unroll
  for (int j = j0; j < j1; ++j) {
    const int blk = min(wave + NWI * j, SLOT_BLOCKS - 1);
    const int u = min(blk * 64 + lane, SLOT_U4 - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(slot + u * 16),
                                     (lds_void*)(buf + blk * 1024), 16, 0, AUX);
  }
}

// Overlapped schedule: wait until the chunk-parallel kernel running beside
// the carry has flagged a slot as stored.  The poll is bounded (`limit`
// polls); false if it gave up.
__device__ __forceinline__ bool wait_ready(const int* flag, int limit) {
  for (int it = 0; it < limit; ++it) {
    if (__builtin_amdgcn_readfirstlane(__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0)
      return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// 16-byte operand read of logical piece `piece` of swizzled row `row`.
__device__ __forceinline__ f16x8 swz_read(const unsigned char* base, int row, int row_bytes, int piece) {
  return *reinterpret_cast<const f16x8*>(base + row * row_bytes + ((piece ^ (row & 7)) << 4));
}


// Slot prefetch split into three groups issued between the products of a
// chunk, so the vector-memory pipe drains while the matrix cores work.
constexpr int PF1 = 6, PF2 = 12;

// One workgroup per CU (its LDS footprint), so one wave per SIMD: telling the
// compiler lets it schedule for latency with the full register file.
//
// CW = state columns per wave: 16 (two workgroups per unit, 64 columns each)
// or 32 (one workgroup per unit; each wave runs its two 16-column tiles
// through the same operand reads, so a slot is staged once per unit and each
// operand read serves twice the columns, at twice the matrix work per wave).
// A column's arithmetic is the same in both.
template <int CW>
__global__ __launch_bounds__(NTI) __attribute__((amdgpu_waves_per_eu(1, 1))) void inter_kernel(Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NCT = CW / 16;                   // 16-column tiles per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  // CW = 16: workgroups 16g + j and 16g + 8 + j (j < 8) are the two column
  // halves of unit 8g + j: with workgroups dealt round-robin over the 8
  // XCDs, both halves of a unit run on one XCD and share its L2 for the slot
  // reads.  CW = 32: workgroup u is unit u.
  int unit, half;
  if constexpr (NCT == 1) {
    const int grp = blockIdx.x >> 4, within = blockIdx.x & 15;
    half = within >> 3;
    unit = 8 * grp + (within & 7);
  } else {
    half = 0;
    unit = blockIdx.x;
  }
  if (unit >= p.N * p.HV) return;
  // Overlapped schedule's repair launch: only units whose 32-column carry
  // gave up are redone.
  if (NCT == 1 && p.status && p.status[unit] == 0) return;
  const int n = unit / p.HV;
  const int hv = unit - n * p.HV;
  int64_t tok0;
  int len;
  seq_range(p, n, tok0, len);
  const int nch = (len + C - 1) / C;
  // This launch covers the sequence's chunks whose slots lie in the window
  // [w0, w1); the state enters from initial_state at chunk 0 and otherwise
  // from final_state, where the previous window left it.  An empty
  // sequence passes its state through in the first window.
  const int64_t base = slot_base(p, n);
  const int c_lo = int(max(int64_t(0), p.w0 - base));
  const int c_hi = int(min(int64_t(nch), p.w1 - base));
  if (c_lo >= c_hi && !(nch == 0 && p.w0 == 0)) return;
  // Workspace slot of chunk c: (hv, base + c - w0).
  auto slot_of = [&](int c) {
    return p.ws + (int64_t(hv) * p.wslots + (base + c - p.w0)) * WS_SLOT;
  };
  // Overlapped schedule (32-column form): the slots are being stored while
  // this kernel runs; each is read only after its ready flag is seen, with
  // device-scope loads.
  constexpr int SAUX = NCT == 2 ? AUX_DEV : 0;
  const int* flag_base = (NCT == 2 && p.flags) ? p.flags + ((base - p.w0) * p.HV + hv) : nullptr;
  auto flagged = [&](int c) {
    (void)c;
    return NCT == 2 && flag_base != nullptr;
  };
  unsigned char* sv = smem + OFF_V + wave * (C * CW * 2);   // NCT v tiles of 2 KB
  const int c0 = half * VT + wave * CW;          // first state column of this wave

  f32x4 S[NCT][8];                               // rows 16rt + 4gq + r of column c0 + 16t + l16
  const float* s_in = c_lo > 0 ? p.sfin : p.s0;
  if (s_in) {   // one branch around all the loads, so they are in flight together
    const float* s0 = s_in + (int64_t(n) * p.HV + hv) * KD * KD;
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[t][rt][r] = s0[(16 * rt + 4 * gq + r) * KD + c0 + 16 * t + l16];
  } else {
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) S[t][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // rdy: the next chunk's slot is known to be stored.  A wave that gives up
  // waiting (gave) waits no more and records it in its own word of abort_w
  // (set only from 0 to 1); after the last barrier every wave reads the same
  // verdict.  Data read after giving up may be stale: the unit's outputs are
  // then redone by the repair launch, and it writes no final state.
  int rdy = 1;
  bool gave = false;
  int* abort_w = reinterpret_cast<int*>(smem + off_abort(CW));
  if constexpr (NCT == 2) {
    if (lane == 0) abort_w[wave] = 0;
  }
  auto wait_for = [&](int c) __attribute__((always_inline)) {
    if (!gave && !wait_ready(flag_base + int64_t(c) * p.HV, p.wait_limit)) {
      gave = true;
      if (lane == 0) abort_w[wave] = 1;
    }
  };
  if (c_lo < c_hi) {
    if (flagged(c_lo)) wait_for(c_lo);
    rdy = flagged(c_lo + 1) ? 0 : 1;
    load_slot_part<SAUX>(smem, slot_of(c_lo), wave, lane, 0, BLOCKS_PER_WAVE);
#pragma unroll
    for (int t = 0; t < NCT; ++t)
      load_v_lds(sv + t * 2048, p, tok0 + int64_t(c_lo) * C, min(C, len - c_lo * C), hv, c0 + 16 * t, lane);
  }
  __builtin_amdgcn_s_waitcnt(WAIT_ALL);
  lds_barrier();

  for (int c = c_lo; c < c_hi; ++c) {
    // The flag of the chunk after next, polled a chunk ahead of its use.  The
    // load is unconditional (an input word stands in where no flag is
    // needed) so that the wait for it stays counted exactly and implied by
    // the one at the end of the chunk.
    bool need2 = false;
    int fl2 = 1;
    if constexpr (NCT == 2) {
      need2 = c + 2 < c_hi && flagged(c + 2);
      const int* fa = need2 ? flag_base + int64_t(c + 2) * p.HV : reinterpret_cast<const int*>(p.v);
      fl2 = __hip_atomic_load(fa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int nvalid = min(C, len - c * C);
    const int64_t trow = tok0 + int64_t(c) * C;
    const unsigned char* cur = smem + ((c - c_lo) & 1) * BUF_BYTES;
    unsigned char* nbuf = smem + ((c - c_lo + 1) & 1) * BUF_BYTES;   // last read in the previous chunk
    // The next chunk's inputs, prefetched unconditionally (the window's last
    // chunk re-reads its own, which nothing uses) so the body has no branches.
    const int cn = min(c + 1, c_hi - 1);
    const unsigned char* nslot = slot_of(cn);

    const unsigned char* sW = cur + WS_W;
    const unsigned char* sQg = cur + WS_QG;
    const unsigned char* sKgT = cur + WS_KGT;
    const unsigned char* sAqk = cur + WS_AQK;
    const unsigned char* sA = cur + WS_A;
    const float* sGam = reinterpret_cast<const float*>(cur + WS_GAM);

    // v as the B operand of U = A v: tokens 32s + 8gq + e of column `col`.
    // Rows past the chunk's end hold copies of its last row (finite) and
    // need no masking: their beta is zero, so their columns of A are exact
    // zeros.
    f16x8 Vv[NCT][2];
#pragma unroll
    for (int t = 0; t < NCT; ++t) read_v_operand(sv + t * 2048, l16, gq, Vv[t]);
    // This wave's v slot is free once its reads are done: fetch the next
    // chunk's, then the first part of the next slot.
    __builtin_amdgcn_s_waitcnt(WAIT_LDS);
    if (!rdy && cn != c) wait_for(cn);
#pragma unroll
    for (int t = 0; t < NCT; ++t)
      load_v_lds(sv + t * 2048, p, tok0 + int64_t(cn) * C, min(C, len - cn * C), hv, c0 + 16 * t, lane);
    load_slot_part<SAUX>(nbuf, nslot, wave, lane, 0, PF1);

    // Contraction orders: for products with S the channel index of k-slot
    // (gq, e) is 32s + 4gq + e (e < 4) or 32s + 16 + 4gq + (e - 4), which is
    // exactly where the float32 S accumulator already holds it; products with
    // Vnew use the same permutation over tokens.  The workspace stores W, Qg,
    // Kg^T and Aqk in that order, so each operand is one 16-byte read.
    //
    // With one wave per SIMD nothing else hides LDS latency, so every
    // product's operands are read in one burst a product ahead of its MFMAs;
    // sched_barrier keeps the compiler from re-interleaving them one by one.
    f16x8 oA[6], oW[16];
#pragma unroll
    for (int mt = 0, i = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) oA[i++] = swz_read(sA, 16 * mt + l16, 128, 4 * s + gq);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oW[4 * s + mt] = swz_read(sW, 16 * mt + l16, 256, 4 * s + gq);
    // S as the fp16 operand of the products with S; then, in the same pass
    // over the accumulators, the decay e^{G_last} S of the state update.
    f16x8 Sh[NCT][4];
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Sh[t][s][r] = (_Float16)S[t][2 * s][r];
          Sh[t][s][4 + r] = (_Float16)S[t][2 * s + 1][r];
        }
    {
      f32x4 gam[8];
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) gam[rt] = *reinterpret_cast<const f32x4*>(sGam + 16 * rt + 4 * gq);
#pragma unroll
      for (int t = 0; t < NCT; ++t)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[t][rt][r] *= gam[rt][r];
    }
    __builtin_amdgcn_sched_barrier(0);

    // U = A v, then Vnew = U + (-W) S; the token tiles are independent
    // accumulation chains.
    f32x4 Vn[NCT][4];
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Vn[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int mt = 0, i = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s, ++i)
#pragma unroll
        for (int t = 0; t < NCT; ++t)
          Vn[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oA[i], Vv[t][s], Vn[t][mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_slot_part<SAUX>(nbuf, nslot, wave, lane, PF1, PF2);
    f16x8 oQ[16];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) oQ[4 * s + mt] = swz_read(sQg, 16 * mt + l16, 256, 4 * s + gq);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < NCT; ++t)
          Vn[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oW[4 * s + mt], Sh[t][s], Vn[t][mt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_slot_part<SAUX>(nbuf, nslot, wave, lane, PF2, BLOCKS_PER_WAVE);
    f16x8 oQK[6];
#pragma unroll
    for (int mt = 0, i = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s) oQK[i++] = swz_read(sAqk, 16 * mt + l16, 128, 4 * s + gq);
    // Kg^T for the state update, read here so that its LDS latency hides
    // behind the O products (measured 1% faster in the overlapped schedule,
    // neutral in the sequential one).
    f16x8 oK[16];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) oK[8 * s + rt] = swz_read(sKgT, 16 * rt + l16, 128, 4 * s + gq);
    __builtin_amdgcn_sched_barrier(0);
    // O^T = S^T Qg^T + Vnew^T Aqk^T: the same operands as O = Qg S + Aqk Vnew
    // with their roles swapped, so each lane ends up holding four adjacent
    // columns of one token and writes them with one 8-byte store.
    f32x4 Ot[NCT][4];
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) Ot[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int t = 0; t < NCT; ++t)
          Ot[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Sh[t][s], oQ[4 * s + mt], Ot[t][mt], 0, 0, 0);
    f16x8 Vh[NCT][2];
#pragma unroll
    for (int t = 0; t < NCT; ++t)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Vh[t][s][r] = (_Float16)Vn[t][2 * s][r];
          Vh[t][s][4 + r] = (_Float16)Vn[t][2 * s + 1][r];
        }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mt = 0, i = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s <= (mt >> 1); ++s, ++i)
#pragma unroll
        for (int t = 0; t < NCT; ++t)
          Ot[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Vh[t][s], oQK[i], Ot[t][mt], 0, 0, 0);
    // S = (e^{G_last} S) + Kg^T Vnew; eight independent row tiles per column tile.
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int t = 0; t < NCT; ++t)
          S[t][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(oK[8 * s + rt], Vh[t][s], S[t][rt], 0, 0, 0);
    // Buffer stores against a range of exactly the chunk's valid rows: the
    // hardware drops the rows past the end, with no branch.
    {
      const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
          p.o + (trow * p.HV + hv) * KD, 0, nvalid * p.HV * KD * 2, BUF_RSRC_WORD3);
#pragma unroll
      for (int t = 0; t < NCT; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int tk = 16 * mt + l16;
          const u32x2_t w = {pack_bf16(Ot[t][mt][0], Ot[t][mt][1]), pack_bf16(Ot[t][mt][2], Ot[t][mt][3])};
          __builtin_amdgcn_raw_buffer_store_b64(w, orsrc, (tk * p.HV * KD + c0 + 16 * t + 4 * gq) * 2, 0, 0);
        }
    }
    // The next chunk's slot and v tiles must have landed before anyone reads
    // them.  They were issued before this chunk's 4 NCT o stores, and exactly
    // those stores follow them, so waiting until at most that many memory
    // operations remain covers the loads without waiting for the stores.
    __builtin_amdgcn_s_waitcnt(NCT == 1 ? WAIT_VM4 : WAIT_VM8);
    if constexpr (NCT == 2) rdy = need2 ? __builtin_amdgcn_readfirstlane(fl2) : 1;
    lds_barrier();
  }
  // A unit whose carry gave up waiting leaves its outputs to the repair
  // launch: no final state (so an initial state stored in the same place
  // is still intact there), and its status word set.
  if constexpr (NCT == 2) {
    const int4 a = *reinterpret_cast<const int4*>(abort_w);
    if ((a.x | a.y | a.z | a.w) != 0) {
      if (tid == 0) __hip_atomic_store(p.status + unit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }

  float* sf = p.sfin + (int64_t(n) * p.HV + hv) * KD * KD;
#pragma unroll
  for (int t = 0; t < NCT; ++t)
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sf[(16 * rt + 4 * gq + r) * KD + c0 + 16 * t + l16] = S[t][rt][r];
}

// Raise a kernel's dynamic-LDS limit, once per device (the attribute is a
// property of the function on the current device).
constexpr int kMaxDevices = 64;
template <typename Kern>
int set_lds(Kern kern, int bytes, std::atomic<bool> (&done)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  if (!done[dev].load(std::memory_order_acquire)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            bytes) != hipSuccess)
      return KDA_ERR_HIP;
    done[dev].store(true, std::memory_order_release);
  }
  return KDA_OK;
}

int64_t slots_per_head(int64_t tokens, int64_t nseq) { return tokens / C + nseq + 1; }

// Ready flags of the overlapped schedule: one int per (value head, slot),
// after the slots, then one status int per (sequence, value head) unit, in
// 256-byte units.
size_t flag_bytes(int64_t nslots, int64_t HV, int64_t nseq) {
  return (size_t((nslots + nseq) * HV) * 4 + 255) & ~size_t(255);
}

// Polls a 32-column carry makes for one flag before it gives up (about
// 0.9 ms, against waits of tens of us in normal running; a unit that gives
// up is redone by the sequential carry after the join).  Settable for tests
// (kda_prefill_overlap_wait_limit).
constexpr int kWaitLimit = 1 << 14;
std::atomic<int> g_wait_limit{kWaitLimit};

using kda::device_cus;

// The split form runs over windows of chunk slots: the chunk-parallel kernel
// fills the window's slots of every value head, then the carry kernel walks
// them, and the next window reuses the same workspace region; the state
// crosses windows through final_state.  Windows bound the workspace (2 GiB
// here, one window for all but very long inputs; the allocation-free entry
// point uses its 64 MiB array).  Measured on MI355X: windows sized to stay in
// the 256 MB last-level cache (96 MB at 96 value heads, T = 8192) made the
// call 14% slower, the per-window ramp and tail of the two kernels costing
// more than the cache residency saves.
#ifndef KDA_WINDOW_BYTES
#define KDA_WINDOW_BYTES (2048ll << 20)
#endif
constexpr int64_t kWindowBytes = KDA_WINDOW_BYTES;

// Slots per value head in one window of at most `bytes` of workspace (at
// least one slot; 0 if even one slot per value head does not fit).
int64_t window_slots(int64_t nslots, int64_t HV, int64_t bytes) {
  const int64_t w = bytes / (HV * WS_SLOT);
  return w < nslots ? w : nslots;
}

// Overlapped split schedule.  The sequential schedule runs the
// chunk-parallel kernel on every CU, then the carry on two workgroups per
// unit; the carry walks its chunks one after another and leaves most of its
// CUs' arithmetic idle.  Here one chunk-kernel launch covers the chunk rows
// [0, rs) (a row: one chunk of every unit) on every CU, then its first keep
// workgroups (about CUs - units, see overlap_keep) go on to [rs, rows) while
// the others leave, and the carry -- one workgroup per unit with 32 state
// columns per wave (inter_kernel<32>), on a second stream -- takes their
// CUs, waiting for each slot to be flagged.  rs is chosen so that the
// chunk kernel and the carry end together: with t_item the chunk kernel's
// time per item per CU and t_step the carry's time per chunk while both run,
//   (rows - rs) * units * t_item / keep = rows * t_step.
// t_step / t_item = 0.357 is the ratio whose split row timed fastest on
// MI355X at B=1, H=HV=96, T=8192, each ratio in a process of its own (51
// of 128 rows: 717.3-718.1 us; 49 rows 718.0-719.7, 54 rows 721.2-722.7,
// 57 rows 729.2-730.6); against 0.345 it ties from 128 to 191 units, is
// 4-5 us faster at 96 units over 128 rows (one or two sequences) and 2 us
// slower over 64 rows, and 0.30 and 0.40 are slower still.  An earlier form
// in two chunk launches, the carry
// started at the first one's end, measured 11 us slower (the launch
// boundary's gaps and the first launch's tail).
#ifndef KDA_OVERLAP_RATIO
#define KDA_OVERLAP_RATIO 0.357
#endif

struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex m;   // one call's fork-join sequence at a time
};

// The calling device's second stream and its two events, made on first use
// and kept for the life of the process (null if the runtime refuses).  They
// are not made while `stream` is being captured into a graph (making a
// stream there can invalidate the capture): such a call runs the sequential
// schedule, and calls after one uncaptured overlapped call capture the
// overlap.
SideStream* side_stream(hipStream_t stream) {
  static std::atomic<SideStream*> side[kMaxDevices];
  static std::mutex make;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream* s = side[dev].load(std::memory_order_acquire);
  if (s) return s;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(make);
  s = side[dev].load(std::memory_order_acquire);
  if (s) return s;
  s = new SideStream;
  if (hipStreamCreateWithFlags(&s->stream, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&s->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&s->join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;   // the partial object is leaked once; calls fall back to the sequential schedule
  }
  side[dev].store(s, std::memory_order_release);
  return s;
}

// Chunk rows of the overlapped schedule: with every sequence T tokens long
// (no cu_seqlens) a row is chunk c of all N sequences (the chunk kernel
// enumerates its items chunk-major); with cu_seqlens and one sequence a row
// is one slot of the window.  Rows of the other packed inputs are not
// formed, so they run sequentially.
int64_t overlap_row_count(const Params& p) {
  if (!p.cu) return (int64_t(p.T) + C - 1) / C;
  return p.N == 1 ? p.nslots : 0;
}

// Workgroups of the overlapped chunk kernel that stay after the split row.
// The others leave and the carry's workgroups take their CUs; their count is
// rounded up to a multiple of 32 (8 XCDs x 4 shader engines) so that every
// shader engine frees at least as many CUs as the carry places on it,
// however the dispatcher spreads the two kernels over them.  Freeing
// exactly `units` CUs, 48, 176 and 191 units measured 23-42% slower at
// T = 8192 (708 against 499 us at 48): a few carry workgroups found no free
// CU where they were placed and waited for the chunk kernel's end.  Letting
// the first workgroups leave instead of the last measured 8 us slower at 96
// units.
int64_t overlap_keep(int64_t units, int64_t cus) { return cus - (units + 31) / 32 * 32; }

// Split row of the overlapped schedule, or 0 where it does not apply: rows
// as above, one workspace window with room for the flags, 48 to CUs - 32
// (sequence, value head) units, and at least 48 chunk rows, or at least 24
// where the sequential carry's two workgroups per unit exceed the CUs.
// Measured on MI355X at T = 8192 against the sequential schedule: 16 and 32
// value heads 33% and 7% slower (the 32-column carry is slower than the
// two-workgroup one and little chunk work is left to overlap), 48 to 191
// value heads 5% to 17% faster; at 96 value heads, 40 rows 1% and 64 rows
// 4% faster, 32 rows 2% slower (64 units 6%, 128 units 2%, 48 units 21%
// slower); with 136 to 191 units, 24 to 40 rows 3% to 14% faster.
int64_t overlap_rows(const Params& p) {
  const int64_t units = int64_t(p.N) * p.HV;
  const int64_t cus = device_cus();
  const int64_t rows = overlap_row_count(p);
  if (!p.flags || p.wslots < p.nslots || units < 48 || units > cus - 32) return 0;
  if (rows < 48 && !(rows >= 24 && 2 * units > cus)) return 0;
  const double keep = double(overlap_keep(units, cus));
  int64_t rs = int64_t(double(rows) * (1.0 - KDA_OVERLAP_RATIO * keep / double(units)));
  if (rs < 1) rs = 1;
  if (rs > rows - 1) rs = rows - 1;
  return rs;
}

// Clears the overlapped schedule's flags and status words.
__global__ void clear_flags_kernel(int* f, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) f[i] = 0;
}

int launch_overlapped(Params p, int64_t rs, hipStream_t stream, SideStream* side) {
  static std::atomic<bool> pub_set[kMaxDevices], inter_set[kMaxDevices], rep_set[kMaxDevices];
  if (set_lds(&intra_kernel<false, true>, SPLIT_LDS, pub_set) != KDA_OK) return KDA_ERR_HIP;
  if (set_lds(&inter_kernel<32>, inter_lds(32), inter_set) != KDA_OK) return KDA_ERR_HIP;
  if (set_lds(&inter_kernel<16>, inter_lds(16), rep_set) != KDA_OK) return KDA_ERR_HIP;
  const int64_t units = int64_t(p.N) * p.HV;
  const int64_t cus = device_cus();
  p.w0 = 0;
  p.w1 = p.nslots;
  p.cmajor = p.cu ? 0 : 1;
  p.status = p.flags + p.nslots * p.HV;
  p.wait_limit = g_wait_limit.load(std::memory_order_relaxed);
  // The chunk kernel: items of the first rs rows over every CU, the rest over
  // the workgroups that stay; the carry takes the CUs of those that leave.
  Params chunks = p;
  chunks.phase2_lo = rs * (p.cmajor ? units : p.HV);
  chunks.phase2_wgs = int(overlap_keep(units, cus));
  Params repair = p;      // the sequential carry, for the units that gave up
  repair.flags = nullptr;
  repair.cmajor = 0;
  const int64_t nclear = p.nslots * p.HV + units;
  std::lock_guard<std::mutex> lock(side->m);
  hipLaunchKernelGGL(clear_flags_kernel, dim3(unsigned((nclear + 1023) / 1024)), dim3(1024), 0, stream, p.flags,
                     nclear);
  int st = launch_status();
  if (st != KDA_OK) return st;
  if (hipEventRecord(side->fork, stream) != hipSuccess) return KDA_ERR_HIP;
  hipLaunchKernelGGL((intra_kernel<false, true>), dim3(unsigned(cus)), dim3(NT), SPLIT_LDS, stream, chunks);
  st = launch_status();
  if (st != KDA_OK) return st;
  // The carry is enqueued after the chunk kernel and waits only for the
  // flags' clearing, so its workgroups get the CUs the chunk kernel leaves.
  // (A runtime that runs the two one after the other runs the carry either
  // after the chunk kernel, where it never waits, or before it, where every
  // unit gives up after its bounded wait and the repair launch redoes it.)
  if (hipStreamWaitEvent(side->stream, side->fork, 0) != hipSuccess) return KDA_ERR_HIP;
  hipLaunchKernelGGL(inter_kernel<32>, dim3(unsigned(units)), dim3(NTI), inter_lds(32), side->stream, p);
  st = launch_status();
  if (st != KDA_OK) return st;
  if (hipEventRecord(side->join, side->stream) != hipSuccess || hipStreamWaitEvent(stream, side->join, 0) != hipSuccess)
    return KDA_ERR_HIP;
  hipLaunchKernelGGL(inter_kernel<16>, dim3(unsigned(16 * ((units + 7) / 8))), dim3(NTI), inter_lds(16), stream,
                     repair);
  return launch_status();
}

// Launch the split form over windows of p.wslots slots (p.ws holds
// p.wslots slots per value head), overlapped where that applies.
int launch(Params p, hipStream_t stream) {
  if (const int64_t rs = overlap_rows(p)) {
    if (SideStream* side = side_stream(stream)) return launch_overlapped(p, rs, stream, side);
  }
  static std::atomic<bool> intra_set[kMaxDevices], inter_set[kMaxDevices];
  if (set_lds(&intra_kernel<false>, SPLIT_LDS, intra_set) != KDA_OK) return KDA_ERR_HIP;
  if (set_lds(&inter_kernel<16>, inter_lds(16), inter_set) != KDA_OK) return KDA_ERR_HIP;
  if (p.wslots < 1) return KDA_ERR_WORKSPACE;
  if (p.wslots * p.HV > 0x7fffffff - 0x10000) return KDA_ERR_SHAPE;   // 32-bit item ids in the intra kernel
  const int64_t units = int64_t(p.N) * p.HV;
  const int64_t inter_blocks = 16 * ((units + 7) / 8);   // two column halves per unit
  if (inter_blocks > 0x7fffffff) return KDA_ERR_SHAPE;
  for (int64_t w0 = 0; w0 < p.nslots; w0 += p.wslots) {
    p.w0 = w0;
    p.w1 = w0 + p.wslots < p.nslots ? w0 + p.wslots : p.nslots;
    const int64_t items = (p.w1 - p.w0) * p.HV;
    p.flags = nullptr;
    p.status = nullptr;
    p.cmajor = 0;
    p.phase2_wgs = 0;
    const int64_t intra_blocks = items < device_cus() ? items : device_cus();
    hipLaunchKernelGGL(intra_kernel<false>, dim3(unsigned(intra_blocks)), dim3(NT), SPLIT_LDS, stream, p);
    int st = launch_status();
    if (st != KDA_OK) return st;
    hipLaunchKernelGGL(inter_kernel<16>, dim3(unsigned(inter_blocks)), dim3(NTI), inter_lds(16), stream, p);
    st = launch_status();
    if (st != KDA_OK) return st;
  }
  return KDA_OK;
}

// Fused form: one workgroup per (sequence, value head); no workspace.
int launch_fused(const Params& p, hipStream_t stream) {
  static std::atomic<bool> fused_set[kMaxDevices];
  if (set_lds(&intra_kernel<true>, FUSED_LDS, fused_set) != KDA_OK) return KDA_ERR_HIP;
  const int64_t units = int64_t(p.N) * p.HV;
  if (units > 0x7fffffff) return KDA_ERR_SHAPE;
  hipLaunchKernelGGL(intra_kernel<true>, dim3(unsigned(units)), dim3(NT), FUSED_LDS, stream, p);
  return launch_status();
}

// Metadata checks shared by both forms; fills everything but the workspace.
int prepare(const void* q, const void* k, const void* v, const float* g, const void* beta,
            const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
            int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd, void* o, float* final_state,
            Params& p) {
  // HV <= 65535 keeps the kernels' 32-bit offsets within a chunk in range.
  if (B < 1 || T < 0 || H < 1 || HV < 1 || HV > 65535 || HV % H != 0) return KDA_ERR_SHAPE;
  if (!final_state || (T > 0 && (!q || !k || !v || !g || !beta || !o))) return KDA_ERR_NULL;
  if (Kd != KD || Vd != KD) return KDA_ERR_UNSUPPORTED;
  if (cu_seqlens && (B != 1 || num_seqs < 1)) return KDA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(o) ||
      !aligned16(final_state) || (initial_state && !aligned16(initial_state)))
    return KDA_ERR_ALIGN;
  const int64_t nseq = cu_seqlens ? num_seqs : B;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.g = g;
  p.beta = static_cast<const uint16_t*>(beta);
  p.s0 = initial_state;
  p.cu = cu_seqlens;
  p.o = static_cast<uint16_t*>(o);
  p.sfin = final_state;
  p.ws = nullptr;
  p.nslots = slots_per_head(int64_t(B) * T, nseq);
  p.w0 = 0;
  p.w1 = p.nslots;
  p.wslots = p.nslots;
  p.flags = nullptr;
  p.cmajor = 0;
  p.phase2_lo = 0;
  p.phase2_wgs = 0;
  p.status = nullptr;
  p.wait_limit = 0;
  p.T = T;
  p.H = H;
  p.HV = HV;
  p.N = int(nseq);
  return KDA_OK;
}

}  // namespace

extern "C" size_t kda_chunk_prefill_workspace_size(int32_t B, int32_t T, int32_t H, int32_t HV,
                                                   int32_t Kd, int32_t Vd, int32_t num_seqs) {
  (void)H;
  if (B < 1 || T < 0 || HV < 1 || Kd != KD || Vd != KD) return 0;
  const int64_t nseq = num_seqs > 0 ? num_seqs : B;
  const int64_t nslots = slots_per_head(int64_t(B) * T, nseq);
  const int64_t w = window_slots(nslots, HV, kWindowBytes);
  const size_t slots = size_t((w > 0 ? w : 1) * HV) * WS_SLOT;
  return w == nslots ? slots + flag_bytes(nslots, HV, nseq) : slots;
}

// The partition kda_chunk_prefill runs.  The fused form walks each
// (sequence, value head) unit's chunks on one compute unit with no workspace;
// the split form spreads the chunk-local work over the whole chip and pays
// the workspace round trip and a second, latency-bound kernel.  Measured on
// MI355X (256 compute units, T = 1024 to 8192): the fused form takes 0.74 to
// 0.93 of the split form's time from 192 units up, and 2x at 96 units, so it
// is chosen from 3/4 as many units as compute units.  Both give the same
// results bit for bit.
bool use_fused(int64_t units) { return units * 4 >= int64_t(device_cus()) * 3; }

// Checks the caller's workspace and points p at it: windows of as many slots
// as it holds, up to the one window kda_chunk_prefill_workspace_size sizes.
// Both the split and the automatic entry point check it, so a call's errors
// do not depend on the partition the device picks.
int take_workspace(Params& p, int32_t B, int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                   void* workspace, size_t workspace_bytes) {
  if (!aligned16(workspace)) return KDA_ERR_ALIGN;
  if (!workspace) return KDA_ERR_NULL;
  const size_t per = size_t(HV) * WS_SLOT;
  if (workspace_bytes < per) return KDA_ERR_WORKSPACE;
  const size_t full = kda_chunk_prefill_workspace_size(B, T, H, HV, Kd, Vd, p.N);
  const int64_t w = window_slots(p.nslots, HV, kWindowBytes);
  const size_t slots = size_t(w > 0 ? w : 1) * per;
  p.ws = static_cast<unsigned char*>(workspace);
  p.wslots = int64_t((workspace_bytes < slots ? workspace_bytes : slots) / per);
  // The flags follow the slots when one window holds every slot and the
  // workspace has room for them (what the size query returns).
  p.flags = (p.wslots == p.nslots && full > slots && workspace_bytes >= full)
                ? reinterpret_cast<int*>(p.ws + slots) : nullptr;
  return KDA_OK;
}

extern "C" int kda_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                                 const void* beta, const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                 int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                 void* o, float* final_state, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  Params p;
  const int st = prepare(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, HV, Kd, Vd, o,
                         final_state, p);
  if (st != KDA_OK) return st;
  const int wst = take_workspace(p, B, T, H, HV, Kd, Vd, workspace, workspace_bytes);
  if (wst != KDA_OK) return wst;
  return use_fused(int64_t(p.N) * HV) ? launch_fused(p, as_stream(stream)) : launch(p, as_stream(stream));
}

extern "C" int kda_chunk_prefill_partition(int32_t B, int32_t HV, int32_t num_seqs) {
  if (B < 1 || HV < 1 || HV > 65535) return -KDA_ERR_SHAPE;
  const int64_t nseq = num_seqs > 0 ? num_seqs : B;
  return use_fused(nseq * HV) ? KDA_PARTITION_FUSED : KDA_PARTITION_SPLIT;
}

extern "C" int kda_chunk_prefill_split(const void* q, const void* k, const void* v, const float* g,
                                       const void* beta, const float* initial_state,
                                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                       int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                       void* o, float* final_state, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  Params p;
  const int st = prepare(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, HV, Kd, Vd, o,
                         final_state, p);
  if (st != KDA_OK) return st;
  const int wst = take_workspace(p, B, T, H, HV, Kd, Vd, workspace, workspace_bytes);
  if (wst != KDA_OK) return wst;
  return launch(p, as_stream(stream));
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the workspace is a file-scope device array.  Its
// name is a host-side stand-in in host code, so its device address is looked
// up once per device (hipGetSymbolAddress, with that device current) and only
// that address is passed to the kernels.  Every call on a device shares the
// array: calls that overlap on one device race.  The kernels write every slot
// they read in the same call, so nothing needs clearing between calls.  The
// prefill runs in windows of as many chunk slots as the array holds, so any
// size fits whose value heads take one slot each (HV <= 1016).
constexpr size_t kNoAllocScratch = KDA_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

static void* scratch_address() {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = addr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    addr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

extern "C" int kda_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                                         const void* beta, const float* initial_state,
                                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                         int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                         void* o, float* final_state, void* stream) {
  Params p;
  const int st = prepare(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, HV, Kd, Vd, o,
                         final_state, p);
  if (st != KDA_OK) return st;
  // Windows of as many slots as the static workspace holds.
  p.wslots = window_slots(p.nslots, HV, int64_t(kNoAllocScratch));
  if (p.wslots < 1) return KDA_ERR_WORKSPACE;
  if (use_fused(int64_t(p.N) * HV)) return launch_fused(p, as_stream(stream));   // the array is not touched
  void* ws = scratch_address();
  if (!ws) return KDA_ERR_HIP;
  p.ws = static_cast<unsigned char*>(ws);
  return launch(p, as_stream(stream));
}

extern "C" int kda_chunk_prefill_fused(const void* q, const void* k, const void* v, const float* g,
                                       const void* beta, const float* initial_state,
                                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                                       int32_t T, int32_t H, int32_t HV, int32_t Kd, int32_t Vd,
                                       void* o, float* final_state, void* stream) {
  Params p;
  const int st = prepare(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, B, T, H, HV, Kd, Vd, o,
                         final_state, p);
  if (st != KDA_OK) return st;
  return launch_fused(p, as_stream(stream));
}

extern "C" int32_t kda_prefill_overlap_wait_limit(int32_t polls) {
  const int previous = g_wait_limit.load();
  g_wait_limit.store(polls < 0 ? kWaitLimit : polls);
  return previous;
}
