// Shared device helpers for the DAR attention kernels (gfx950 / CDNA4 only).
//
// Everything here is plumbing: vector types for the MFMA operands, bf16
// conversion, the RoPE cos/sin lookup and the internal launch declarations.
// The method's arithmetic lives in the kernels that include this header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dar.h"

namespace dar {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// Workgroups are handed to the 8 XCDs of an MI355X round-robin by linear id.
constexpr int kNumXcd = 8;

// Workgroup barrier for LDS pipelines: this wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it carries no release fence, which
// would make the wave wait for every outstanding global load too (vmcnt(0)),
// including the direct-to-LDS loads of k-tiles prefetched further ahead.
// Callers wait on vmcnt themselves for the loads the next step reads.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) {
  return x;
}
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  return (bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
}
template <>
__device__ __forceinline__ f16 from_f32<f16>(float x) {
  return (f16)x;  // round to nearest even
}
__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }

// 8-wide MFMA operand of element type T.
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<f16> {
  typedef f16x8 type;
};

// Two fp32 values -> one dword of two bf16 (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 MFMA, fp32 accumulate.  Operand lane layout (wave64):
// lane l supplies row/column (l % 32) and contraction elements
// [8*(l/32), 8*(l/32)+8) of the 16-wide step.  Result register r of lane l
// holds row 8*(r/4) + 4*(l/32) + (r%4), column (l % 32).
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b,
                                               const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// Same shape and lane layout with IEEE fp16 operands.
__device__ __forceinline__ f32x16 mfma32x32x16(const f16x8& a, const f16x8& b,
                                               const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Two fp32 values -> one dword of two fp16 (low half = a).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v;
  v[0] = (f16)a;
  v[1] = (f16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight bf16 (as 4 dwords) -> eight fp16 (as 4 dwords).  Exact for every bf16
// value inside the fp16 normal range.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xffff0000u);
    r[i] = pack_f16x2(lo, hi);
  }
  return r;
}

// RoPE angle lookup.  cos/sin(p * theta_t) is the complex product of a
// coarse entry (p >> 6) and a fine entry (p & 63); both tables are computed
// in fp64 and stored as fp32 (cos, sin) pairs, row length d_k/2.
struct RopeTab {
  const float2* lo;  // [64][half]
  const float2* hi;  // [n_hi][half]
  int half;
};

__device__ __forceinline__ float2 rope_cs(const RopeTab& t, int pos, int k) {
  const float2 a = t.hi[(size_t)(pos >> 6) * t.half + k];
  const float2 b = t.lo[(size_t)(pos & 63) * t.half + k];
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// ----------------------------------------------------------------------------
// Internal launchers (defined in the .hip files, called by the C ABI layer).
// All return hipSuccess or the launch error.

// RoPE tables for positions [0, max_pos], written into lo / hi.
size_t rope_table_bytes(int d_k, long max_pos);
hipError_t launch_rope_tables(float2* lo, float2* hi, int d_k, long max_pos, float base,
                              hipStream_t s);

// Output kinds of the projection GEMM epilogue.
enum OutKind : int {
  kRowMajor = 0,  // out[row, col]                     (h^D, folded weights)
  kHead = 1,      // out[b, head, n, t]                (Q, K_loc, K_glob)
  kHeadT = 2      // out[b, head, t, n]                (V_loc, V_glob)
};

struct GemmSeg {
  const void* Bt;  // operand, [width, K] row-major (column-major weight)
  void* out;
  int width;       // number of output columns in this segment
  int kind;        // OutKind
  int rope;        // rotate (kind == kHead only)
  // Output sequence addressing (every kind): token (b, n) of the GEMM lands at
  // sequence index n + seq_off of a sequence of length ld_seq (ld_seq = 0
  // means the GEMM's own n_seq and seq_off = 0).  This lets the decode append
  // write one token into a ring slot or a latent-cache row, and a prefill
  // chunk write its rows after the prefix's.
  int ld_seq = 0, seq_off = 0;
  // With GemmProblem::row_pos (one token per sequence): where row b lands.
  // kPosFixed: index seq_off; kPosRow: row_pos[b]; kPosRing: row_pos[b] mod ld_seq.
  int pos_mode = 0;
  // kRowMajor only: 1 applies the logistic sigmoid to the fp32 result before
  // it is rounded and stored (the sigmoid-bottleneck variant of h^D)
  int act = 0;
  // kHead / kHeadT: heads of this segment's output ([B, heads, ...]); 0 means
  // GemmProblem::heads.  A one-head segment writes [B, ld, d] (the shared
  // rotary key of the decoupled-RoPE variant).
  int heads = 0;
};
enum PosMode : int { kPosFixed = 0, kPosRow = 1, kPosRing = 2 };

// Element types of GEMM operands and outputs.
enum ElemType : int { kF32 = 0, kBF16 = 1, kF16 = 2 };

struct GemmProblem {
  const void* A;  // [M, K] row-major
  int M, K;
  int a_type, b_type, out_type;  // ElemType of A, of every segment's B, of the outputs
  int nseg;
  GemmSeg seg[4];
  int n_seq;  // rows per sequence (row -> (b, n))
  int heads, d_k, pos0;
  RopeTab rope;
  // Ragged append (n_seq == 1): row b is sequence b's token at position
  // row_pos[b] (device, int32), clamped to [0, pos_max] (the last position the
  // RoPE tables hold); an index past a segment's ld_seq is clamped to its last
  // row.  Null: position pos0 + n.
  const int* row_pos = nullptr;
  int pos_max = 0;
  // Ragged prefill: rows cu[b] .. cu[b+1]-1 (device, int32, n_cu + 1 entries)
  // are sequence b's tokens at positions pos0 + 0, 1, ... (clamped to
  // pos_max); each head-major output holds one [H, len_b, d_k] (V: [H, d_k,
  // len_b]) block per sequence starting at row cu[b] (seg.ld_seq must be 0).
  // Rows outside their sequence (inconsistent cu) are not written.  Null:
  // n_seq rows per sequence.
  const int* cu = nullptr;
  int n_cu = 0;
  // Rows of A between the first rows of consecutive sequences (0: n_seq, the
  // rows packed): GEMM row b n_seq + n reads A row b a_ld_seq + n, e.g. the
  // prefixes of B sequences in a latent cache of a_ld_seq rows each.
  int a_ld_seq = 0;
};

hipError_t launch_project_gemm(const GemmProblem& p, dar_dtype dt, hipStream_t s);

// W_upK^T = W_K^T W_up^T etc. (the fold), fp32 accumulate.
hipError_t launch_fold(const void* W_up, const void* W_KV, void* out, int d, int d_down, int hd,
                       dar_dtype dt, hipStream_t s);

struct PrefillProblem {
  const void *Q, *K_loc, *V_loc, *K_glob, *V_glob;
  void* o;
  int B, N, H, d_k, w;
  // Chunk form (bf16 only): the queries are positions q0 .. N-1 (Q, o hold
  // N - q0 rows), the global arrays hold positions 0 .. N-1 and the local
  // arrays positions loc0 .. N-1.  A whole prefill has q0 = loc0 = 0.
  int q0 = 0, loc0 = 0;
  // Optional [B, H, N] fp32 output (whole prefill only): the natural-log
  // log-sum-exp of each query's scaled scores, log sum_j exp(q_i . k_j / sqrt(d_k)).
  float* lse = nullptr;
  // Decoupled-RoPE variant (whole prefill, bf16): rotary queries QR
  // [B, H, N, d_R] and the shared rotary keys KR [B, N, d_R] extend every
  // score, s = (q . k + qR . kR) / sqrt(d_k + d_R); d_R = 0 otherwise.
  const void* QR = nullptr;
  const void* KR = nullptr;
  int d_R = 0;
  // Ragged prefill (bf16, whole prefills, no lse / rotary part): B sequences,
  // sequence b the rows cu[b] .. cu[b+1]-1 (device, int32) of the packed
  // arrays, each source held as one [H, len_b, d_k] (V: [H, d_k, len_b])
  // block per sequence from row cu[b]; o [T, H d_k]; N is the longest length.
  const int* cu = nullptr;
  int T = 0;
};
hipError_t launch_attn_prefill(const PrefillProblem& p, dar_dtype dt, hipStream_t s);

// Backward of the prefill attention: Q, K_*, V_* in the forward's layouts and
// types (V transposed per head), o and dO [B, N, H*d_k] (bf16 in bf16 mode);
// fp32 gradients [B, H, N, d_k] (dV not transposed); lse, Dd: [B, H, N] fp32
// workspace (per-query log-sum-exp and dO . o).
struct BwdProblem {
  const void *Q, *K_loc, *V_loc, *K_glob, *V_glob, *o, *dO;
  const float* lse_in;  // the forward's natural-log lse [B, H, N], or null
  float *dQ, *dK_loc, *dV_loc, *dK_glob, *dV_glob;
  float *lse, *Dd;
  int B, N, H, d_k, w;
};
size_t attn_backward_workspace_bytes(int B, int N, int H);
hipError_t launch_attn_backward(const BwdProblem& p, dar_dtype dt, hipStream_t s);

struct DecodeProblem {
  const void *q, *K_win, *V_win, *h_D, *W_upK, *W_upV;
  void* o;
  int B, ctx, cap, H, d_k, d_down, w;
  RopeTab rope;
  void* ws;  // workspace after the rope tables
  // Ragged batch: ctx_lens[b] (device, int32) is sequence b's context length,
  // clamped to [1, ctx]; ctx is then the largest.  Null: every sequence has ctx.
  const int* ctx_lens = nullptr;
};
size_t decode_workspace_bytes(const DecodeProblem& p);
// The latent decode's log-sum-exp merge and lift by W_upV over n_chunks latent
// partials (max, sum, acc[d_down]) per (batch, head) and n_win (<= 64) window
// partials (max, sum, acc[d_k]); reads p.W_upV, p.B, p.H, p.d_k, p.d_down,
// writes p.o.
hipError_t launch_decode_combine(const DecodeProblem& p, int n_chunks, const float* part_lat,
                                 const float* part_win, int n_win, hipStream_t s);

// Decode of the decoupled-RoPE variant (attn_decode_drope.hip).
struct DropeDecodeProblem {
  const void *qC, *qR, *K_win, *V_win, *KR, *h_D, *W_upK, *W_upV;
  void* o;
  int B, ctx, cap, H, d_k, d_R, d_down, w;
  void* ws;
};
bool drope_decode_supported(int d_k, int d_R, int d_down);
size_t drope_decode_workspace_bytes(const DropeDecodeProblem& p);
hipError_t launch_attn_decode_drope(const DropeDecodeProblem& p, hipStream_t s);
// Pieces of the cache kernels (fp16 <-> bf16 conversions, positions relative to
// array bases; see cache.hip).
hipError_t launch_latent_cast(const void* h_D, int B, int N, int d_down, int cap, int row0,
                              void* h_D_cache, hipStream_t s, const int* cu = nullptr,
                              int nb = 0);
hipError_t launch_ring_fill(const void* K, const void* Vt, int B, int heads, int d_k, int N,
                            int base, int w, void* K_win, void* V_win, hipStream_t s,
                            const int* lens = nullptr);
hipError_t launch_ring_to_local(const void* K_win, const void* V_win, int B, int heads, int d_k,
                                int w, int base, int p0, int len, void* K, void* Vt,
                                hipStream_t s);
// Decode cache from prefill outputs (fp16 h_D, K_loc, V_loc^T -> bf16 cache).
hipError_t launch_cache_from_prefill(const void* h_D, const void* K_loc, const void* V_loc,
                                     int B, int N, int heads, int d_k, int d_down, int w,
                                     int cap, void* h_D_cache, void* K_win, void* V_win,
                                     hipStream_t s, const int* lens = nullptr);
// The same from packed prompts (dar_project_varlen's layout; prompt starts cu).
hipError_t launch_cache_from_packed(const void* h_D, const void* K_loc, const void* V_loc,
                                    const int* cu, int B, int T, int max_len, int heads, int d_k,
                                    int d_down, int w, int cap, void* h_D_cache, void* K_win,
                                    void* V_win, hipStream_t s);
// Row-major [rows, cols] -> column-major (cache.hip); grid limit rows, cols <= 64 * 65535.
hipError_t launch_pack_weight(const void* W, int rows, int cols, int elem_bytes, void* out,
                              hipStream_t s);
bool decode_supported(int d_k, int d_down);  // d_k in {64,128}, d_down in {32,...,512}
hipError_t launch_attn_decode(const DecodeProblem& p, hipStream_t s);

}  // namespace dar
