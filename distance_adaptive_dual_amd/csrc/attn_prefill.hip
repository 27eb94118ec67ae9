// Fused dual-source causal attention (prefill).
//
// "Dual Dimensionality for Local and Global Attention", Eq. (3)-(4): query i
// attends to every key j <= i; the pair uses the full-state key/value
// (K_loc, V_loc) when i - j < w and the bottleneck key/value (K_glob, V_glob)
// otherwise; o_i = softmax(q_i K_i^T / sqrt(d_k)) V_i.
//
// bf16 mode (gfx950).  The layer's I/O is bf16; Q, K and V arrive as IEEE fp16
// (written so by the projection) and P is rounded to fp16, so both products
// run on fp16 MFMAs with fp32 accumulation.  One workgroup = 128 queries of one (batch, head), four
// waves of 32 queries.  Keys stream in tiles of 64.  Every (query-wave, key
// tile) pair is classified from its distance range [dmin, dmax]:
//   dmax < 0             skipped (causally in the future)
//   dmax < w             local only       (one K/V source)
//   max(dmin, 0) >= w    global only      (one K/V source)
//   otherwise            boundary: scores from both sources, chosen per
//                        element by i - j < w, and two P.V products with the
//                        complementary halves of P.
// The workgroup stages into LDS only the sources some wave needs.  Scores are
// formed transposed, S^T = K Q^T, with 32x32x16 MFMAs so each lane owns one
// query: the running max / sum are per-lane scalars, the row reductions are a
// single exchange between lane halves, and P^T drops straight into the B
// operand of O^T += V^T P^T.  Key rows are fed to the first MFMA in an order
// (bits 2 and 3 of the row index swapped) that makes the eight P values a lane
// holds for one P.V step eight consecutive keys, so V^T is read with one
// 16-byte LDS load per step.  Softmax runs in base 2 with log2(e)/sqrt(d_k)
// folded into the score scale, in fp32.
//
// At d_k = 128, whole prefills whose N is a multiple of 64 run attn_prefill_ring
// instead: eight waves share each key/value tile, which arrives by direct
// loads into a four-stage LDS ring (see there).
//
// fp32 kernel: VALU only, four lanes per query, per-key online softmax; it
// exists for the fp32 mode (1e-4 parity), never rounds to bf16.
#include <math.h>

#include "dar_common.hpp"

namespace dar {

namespace {

constexpr int QT = 128;      // queries per workgroup
constexpr int KT = 64;       // keys per tile
constexpr float kTau = 8.f;  // rescale only when a row max grows by > 2^8 (log2 units)
constexpr float kNegBig = -1e30f;

__device__ __forceinline__ int key_perm(int r) {  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Offset of score register (kb, r) from the lane's first key j0 + 8*lg.
__device__ __forceinline__ constexpr int key_off(int kb, int r) {
  return 32 * kb + 16 * (r >> 3) + (r & 7);
}

// DR > 0 (the decoupled-RoPE variant): a key row holds the content part
// (D) followed by the shared rotary key (DR); values stay D wide.
template <int D, int DR = 0>
struct PassSmem {
  static constexpr int DQ = D + DR;
  static constexpr int KP = DQ + 8;  // fp16 per K row (16 B pad: 4-bank shift per row)
  static constexpr int VP = KT + 8;  // fp16 per V^T row
  f16 k[2][KT * KP];                 // [buffer][key][d]
  f16 v[2][D * VP];                  // [buffer][d][key]
};

// Register staging of one pass: a key tile of one source (K [KT x (D + DR)]
// and V^T [D x KT]), 16-byte chunks spread over the 256 threads.
template <int D, int DR = 0>
struct Stage {
  static constexpr int NCH = KT * D / 8 / 256;         // V chunks per thread
  static constexpr int NCK = KT * (D + DR) / 8 / 256;  // K chunks per thread
  typedef u32x4 KArr[NCK];
  typedef u32x4 VArr[NCH];
  KArr k;
  VArr v;
};

// One 16-byte chunk of K row j (fp16 [N x D] rows, j may lie outside [0, N)):
// through a buffer resource whose range check returns zeros past the rows,
// no branch, while the slice is below 2 GiB; else a guarded load.
template <int D>
__device__ __forceinline__ u32x4 load_k_chunk(const f16* K, int N, int j, int col) {
  if ((long)N * D * 2 < 0x7fffffffL) {
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)K, (short)0, N * D * 2, 0x00020000);
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(rk, (j * D + col) * 2, 0, 0));
  }
  const u32x4 z = {0u, 0u, 0u, 0u};
  return ((unsigned)j < (unsigned)N) ? *(const u32x4*)(K + (size_t)j * D + col) : z;
}

// K and Vt hold positions base .. base+N-1 of one (batch, head) (K [N x D],
// Vt [D x N]); j0 = first position of the tile - base, which may be negative
// for the local arrays of a chunk: rows outside [0, N) read as zeros.
// One 16-byte chunk of a staged key row: the content part from K, the
// rotary part (DR > 0) from KR, the rows of the same positions.
template <int D, int DR>
__device__ __forceinline__ u32x4 load_key_chunk(const f16* K, const f16* KR, int N, int j,
                                                int col) {
  if constexpr (DR > 0) {
    if (col >= D) return load_k_chunk<DR>(KR, N, j, col - D);
  }
  return load_k_chunk<D>(K, N, j, col);
}

template <int D, int DR = 0>
__device__ __forceinline__ void load_pass(Stage<D, DR>& st, const f16* K, const f16* Vt, int N,
                                          int j0, bool vec_ok, const f16* KR = nullptr) {
  constexpr int DQ = D + DR;
  const int tid = threadIdx.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCK; ++i) {
    const int c = tid + 256 * i;
    const int row = c / (DQ / 8), col = (c % (DQ / 8)) * 8;
    st.k[i] = load_key_chunk<D, DR>(K, KR, N, j0 + row, col);
  }
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCH; ++i) {
    const int c = tid + 256 * i;
    const int d = c / (KT / 8), kc = (c % (KT / 8)) * 8;
    if (vec_ok) {
      st.v[i] = *(const u32x4*)(Vt + (size_t)d * N + j0 + kc);
    } else {  // ragged tail, rows outside [0, N), or N not a multiple of 8
      const uint16_t* src = (const uint16_t*)Vt + (size_t)d * N;
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ja = j0 + kc + 2 * e, jb = ja + 1;
        const uint32_t a = (unsigned)ja < (unsigned)N ? src[ja] : 0u;
        const uint32_t b = (unsigned)jb < (unsigned)N ? src[jb] : 0u;
        w4[e] = a | (b << 16);
      }
      st.v[i] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
  }
}

// The two halves of load_pass / store_pass, for staging K and V at different
// times of a pass.
template <int D, int DR = 0>
__device__ __forceinline__ void load_k(typename Stage<D, DR>::KArr& k, const f16* K, int N,
                                       int j0, const f16* KR = nullptr) {
  constexpr int DQ = D + DR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCK; ++i) {
    const int c = tid + 256 * i;
    const int row = c / (DQ / 8), col = (c % (DQ / 8)) * 8;
    k[i] = load_key_chunk<D, DR>(K, KR, N, j0 + row, col);
  }
}

template <int D, int DR = 0>
__device__ __forceinline__ void load_v(typename Stage<D, DR>::VArr& v, const f16* Vt, int N,
                                       int j0, bool vec_ok) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCH; ++i) {
    const int c = tid + 256 * i;
    const int d = c / (KT / 8), kc = (c % (KT / 8)) * 8;
    if (vec_ok) {
      v[i] = *(const u32x4*)(Vt + (size_t)d * N + j0 + kc);
    } else {  // ragged tail, rows outside [0, N), or N not a multiple of 8
      const uint16_t* src = (const uint16_t*)Vt + (size_t)d * N;
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ja = j0 + kc + 2 * e, jb = ja + 1;
        const uint32_t a = (unsigned)ja < (unsigned)N ? src[ja] : 0u;
        const uint32_t b = (unsigned)jb < (unsigned)N ? src[jb] : 0u;
        w4[e] = a | (b << 16);
      }
      v[i] = u32x4{w4[0], w4[1], w4[2], w4[3]};
    }
  }
}

template <int D, int DR = 0>
__device__ __forceinline__ void store_k(const typename Stage<D, DR>::KArr& k, f16* sk) {
  constexpr int KP = PassSmem<D, DR>::KP, DQ = D + DR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCK; ++i) {
    const int c = tid + 256 * i;
    const int row = c / (DQ / 8), col = (c % (DQ / 8)) * 8;
    *(u32x4*)(sk + row * KP + col) = k[i];
  }
}

template <int D, int DR = 0>
__device__ __forceinline__ void store_v(const typename Stage<D, DR>::VArr& v, f16* sv) {
  constexpr int VP = PassSmem<D, DR>::VP;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Stage<D, DR>::NCH; ++i) {
    const int c = tid + 256 * i;
    const int d = c / (KT / 8), kc = (c % (KT / 8)) * 8;
    *(u32x4*)(sv + d * VP + kc) = v[i];
  }
}

template <int D, int DR = 0>
__device__ __forceinline__ void store_pass(const Stage<D, DR>& st, f16* sk, f16* sv) {
  store_k<D, DR>(st.k, sk);
  store_v<D, DR>(st.v, sv);
}

// K fragments of a staged key tile for S^T = K Q^T: kf[kb][st] holds rows
// 32 kb + key_perm(lr) (keys j0 + ...) and dims 16 st + 8 lg .. +8.
template <int D, int DR = 0>
__device__ __forceinline__ void read_kfrags(const f16* sk, f16x8 (&kf)[2][(D + DR) / 16], int lr,
                                            int lg) {
  constexpr int KP = PassSmem<D, DR>::KP;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const f16* base = sk + (32 * kb + key_perm(lr)) * KP + 8 * lg;
#pragma unroll
    for (int st = 0; st < (D + DR) / 16; ++st) kf[kb][st] = *(const f16x8*)(base + 16 * st);
  }
}

// S^T = K Q^T: s[kb][r] is key j0 + 8 lg + key_off(kb, r) of this lane's
// query.  The two 32-key blocks' accumulation chains are interleaved so that
// no MFMA waits on the result of the one just issued.
template <int D, int DR = 0>
__device__ __forceinline__ void mfma_scores(const f16x8 (&kf)[2][(D + DR) / 16],
                                            const f16x8 (&qf)[(D + DR) / 16], f32x16 (&s)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
  for (int st = 0; st < (D + DR) / 16; ++st)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32x32x16(kf[kb][st], qf[st], s[kb]);
}

// Keep mask of Eq. (3) and causality, then the running reference maximum:
// keep iff keep_lo < key_off <= keep_hi.  Softmax is invariant to the
// reference maximum, so it is only moved (and O, l rescaled) when some row's
// maximum exceeds it by more than 2^kTau.
template <int D>
__device__ __forceinline__ void mask_and_max(f32x16 (&s)[2], f32x16 (&o)[D / 32], float& m_ref,
                                             float& l_run, bool masked, int keep_lo, int keep_hi,
                                             float sc) {
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = key_off(kb, r);
        if (!(off > keep_lo && off <= keep_hi)) s[kb][r] = -INFINITY;
      }
  }
  float mt = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
  // the two lane halves hold the two halves of the query's keys
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                   false, false);
  mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc;
  if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTau) != 0) {
    const float m_new = fmaxf(m_ref, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
    m_ref = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
}

// p = 2^(s*sc - m_ref) rounded to fp16 (the P operand), l += the same fp16
// p, and O^T += V^T P^T with the column blocks interleaved per 16-key step.
template <int D>
__device__ __forceinline__ void exp_and_pv(const f16* sv, const f32x16 (&s)[2],
                                           f32x16 (&o)[D / 32], float m_ref, float& l_run,
                                           float sc, int lr, int lg) {
  constexpr int VP = PassSmem<D>::VP;
  // Every V^T fragment of the pass is requested first and arrives while the
  // exponentials run.
  constexpr int VPRE = D / 32;  // column blocks of 32
  f16x8 vf[VPRE][4];
#pragma unroll
  for (int db = 0; db < VPRE; ++db) {
    const f16* vb = sv + (32 * db + lr) * VP + 8 * lg;
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[db][u] = *(const f16x8*)(vb + 16 * u);
  }
  f16x8 pf[4];
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one2 = {(f16)1.f, (f16)1.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + c], sc, -m_ref));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + c + 1], sc, -m_ref));
      const uint32_t pk = pack_f16x2(e0, e1);
      const h2 ph = __builtin_bit_cast(h2, pk);
      l_run = __builtin_amdgcn_fdot2(ph, one2, l_run, false);
      pf[u][c] = ph[0];
      pf[u][c + 1] = ph[1];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int db = 0; db < VPRE; ++db) o[db] = mfma32x32x16(vf[db][u], pf[u], o[db]);
}

// One whole pass of one wave: scores against the staged tile, the keep mask,
// online softmax, and O^T += V^T P^T.
template <int D, int DR = 0>
__device__ __forceinline__ void wave_pass(const f16* sk, const f16* sv,
                                          const f16x8 (&qf)[(D + DR) / 16], f32x16 (&o)[D / 32],
                                          float& m_ref, float& l_run, bool masked, int keep_lo,
                                          int keep_hi, float sc, int lr, int lg) {
  f16x8 kf[2][(D + DR) / 16];
  read_kfrags<D, DR>(sk, kf, lr, lg);
  f32x16 s[2];
  mfma_scores<D, DR>(kf, qf, s);
  mask_and_max<D>(s, o, m_ref, l_run, masked, keep_lo, keep_hi, sc);
  exp_and_pv<D>(sv, s, o, m_ref, l_run, sc, lr, lg);
}

// p = 2^(s*sc - m) for the 16 scores of a lane, rounded to fp16 (the P
// operand of two 16-key steps), and their sum in fp32.
__device__ __forceinline__ void exp_half(const f32x16& s, float sc, float m, f16x8 (&pf)[2],
                                         float& ls) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one2 = {(f16)1.f, (f16)1.f};
  ls = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[8 * u + c], sc, -m));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[8 * u + c + 1], sc, -m));
      const h2 ph = __builtin_bit_cast(h2, pack_f16x2(e0, e1));
      ls = __builtin_amdgcn_fdot2(ph, one2, ls, false);
      pf[u][c] = ph[0];
      pf[u][c + 1] = ph[1];
    }
  }
}

// Half kb of a pass (d_k = 64): scores, mask, maximum, exponentials and P.V
// of keys 32 kb .. 32 kb + 31 of the staged tile.  A pass run as two halves
// keeps only half the score, K and V fragment registers live at a time, which
// fits four waves per SIMD; the reference maximum may move between the halves
// (same rule as a whole pass).
template <int D, int DR = 0>
__device__ __forceinline__ void wave_half(int kb, const f16* sk, const f16* sv,
                                          const f16x8 (&qf)[(D + DR) / 16], f32x16 (&o)[D / 32],
                                          float& m_ref, float& l_run, bool masked, int keep_lo,
                                          int keep_hi, float sc, int lr, int lg) {
  constexpr int KP = PassSmem<D, DR>::KP, VP = PassSmem<D, DR>::VP, NQ = (D + DR) / 16;
  {
    f16x8 kf[NQ];
    {
      const f16* base = sk + (32 * kb + key_perm(lr)) * KP + 8 * lg;
#pragma unroll
      for (int st = 0; st < NQ; ++st) kf[st] = *(const f16x8*)(base + 16 * st);
    }
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int st = 0; st < NQ; ++st) s = mfma32x32x16(kf[st], qf[st], s);
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = key_off(kb, r);
        if (!(off > keep_lo && off <= keep_hi)) s[r] = -INFINITY;
      }
    }
    // p against the current reference maximum; the half's fp16 sum below
    // 2^15 proves every p is far inside fp16 range.  Otherwise (the maximum
    // grew, or the reference is still the initial -1e30) the true maximum is
    // taken, O and l are rescaled and p is recomputed.
    f16x8 pf[2];
    float ls;
    exp_half(s, sc, m_ref, pf, ls);
    if (__builtin_amdgcn_ballot_w64(!(ls < 32768.f)) != 0) {
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt),
                                                       false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * sc;
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      exp_half(s, sc, m_ref, pf, ls);
    }
    l_run += ls;
    // V^T fragments of this half's 32 keys (two 16-key steps u)
    f16x8 vf[D / 32][2];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const f16* vb = sv + (32 * db + lr) * VP + 32 * kb + 8 * lg;
#pragma unroll
      for (int u = 0; u < 2; ++u) vf[db][u] = *(const f16x8*)(vb + 16 * u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mfma32x32x16(vf[db][u], pf[u], o[db]);
  }
}

// What one wave does with one pass (a key tile of one source): whether it has
// any kept pair there, whether the keep mask is needed, and the mask bounds
// relative to the lane's first key j0 + 8 lg.
struct WavePass {
  bool part, masked;
  int keep_lo, keep_hi;
};

__device__ __forceinline__ WavePass wave_pass_info(int j0, int src, int qw0, int wi_last, int qi,
                                                   int lg, int N, int w) {
  WavePass r{false, false, 0, 0};
  const int wdmax = wi_last - j0, wdmin = qw0 - (j0 + KT - 1);
  if (qw0 < N && wdmax >= 0) {
    const bool glob = src == 0;
    r.part = glob ? (wdmax >= w) : (w > 0 && max(wdmin, 0) < w);
    r.masked = (glob ? (wdmin < w) : (wdmin < 0 || wdmax >= w)) || (j0 + KT > N);
    const int base = qi - j0 - 8 * lg;  // distance of key offset 0
    const int lo = glob ? w : 0;
    r.keep_lo = glob ? -1 : base - w;
    r.keep_hi = min(base - lo, N - 1 - j0 - 8 * lg);
  }
  return r;
}

// CHUNK: queries start at p.q0 and the local arrays at p.loc0 (a prefill
// chunk); otherwise both are 0 and compiled in as constants.  LSE: also store
// each query's log-sum-exp in p.lse (whole prefills only).
// DR > 0: the decoupled-RoPE variant (whole prefill only): every key row is
// [content ; shared rotary key] and every query [content ; rotary], so the
// score MFMA chain runs over D + DR; values and the output stay D wide.
template <int D, bool CHUNK, bool LSE, int DR = 0>
__global__ __launch_bounds__(256, (D == 64 && DR == 0) ? 4 : 2) void attn_prefill_f16(
    PrefillProblem p, int nQT, int nPair, int remap, int paired) {
  static_assert(DR == 0 || !CHUNK, "the rotary part covers whole prefills");
  constexpr int NQ = (D + DR) / 16;  // 16-wide steps of the score contraction
  __shared__ PassSmem<D, DR> sm;
  const int H = p.H, BH = p.B * p.H, w = p.w;
  // paired: a workgroup takes query tile nQT-1-pr and then tile pr, so every
  // workgroup streams about the same number of key tiles.  Unpaired: one
  // tile per workgroup, longest first (nPair = nQT).  With remap, all tiles
  // of one (batch, head) stay on one XCD so its K/V prefix is shared through
  // that XCD's L2.
  int pr, bh;
  {
    const int bid = blockIdx.x;
    if (remap) {
      const int x = bid % kNumXcd, k = bid / kNumXcd, G = BH / kNumXcd;
      if (paired) {
        pr = k % nPair;
        bh = (k / nPair) * kNumXcd + x;
      } else {
        pr = k / G;
        bh = (k % G) * kNumXcd + x;
      }
    } else {
      pr = bid / BH;
      bh = bid % BH;
    }
  }
  const int b = bh / H, h = bh % H;
  // Sequence b: N tokens.  Ragged batches (cu, whole prefills only): its rows
  // cu[b] .. cu[b+1]-1 of the packed arrays, clamped into [0, T], each array
  // holding one [H, N, D] block (V: [H, D, N]) per sequence from row cu[b].
  int N = p.N;
  size_t seq0 = 0;
  if (!CHUNK && p.cu != nullptr) {
    const int c0 = min(max(p.cu[b], 0), p.T), c1 = min(max(p.cu[b + 1], c0), p.T);
    N = c1 - c0;
    seq0 = (size_t)c0;
  }
  // Positions: queries q0 .. N-1 (Q and o hold those rows only), keys 0 .. N-1
  // in the global arrays, keys loc0 .. N-1 in the local arrays.
  const int q0 = CHUNK ? p.q0 : 0, loc0 = CHUNK ? p.loc0 : 0, nqr = N - q0, nloc = N - loc0;
  // first element of (batch, head)'s slice of an array of `rows` rows per sequence
  auto slice = [&](int rows) {
    return p.cu != nullptr && !CHUNK ? (seq0 * H + (size_t)h * N) * D : (size_t)bh * rows * D;
  };
  const f16* Qp = (const f16*)p.Q + slice(nqr);
  const f16* Kg = (const f16*)p.K_glob + slice(N);
  const f16* Kl = (const f16*)p.K_loc + slice(nloc);
  const f16* Vg = (const f16*)p.V_glob + slice(N);
  const f16* Vl = (const f16*)p.V_loc + slice(nloc);
  const size_t orow0 = p.cu != nullptr && !CHUNK ? seq0 : (size_t)b * nqr;  // o's first row
  // rotary keys of sequence b (positions 0 .. N-1, every head) and queries
  const f16* KRb = DR > 0 ? (const f16*)p.KR + (size_t)b * N * DR : nullptr;
  const f16* QRp = DR > 0 ? (const f16*)p.QR + (size_t)bh * N * DR : nullptr;
  // array, length, relative tile start and 16-byte V loads for source s at j0
  auto src_len = [&](int s) { return s ? nloc : N; };
  auto src_rel = [&](int s, int j0) { return s ? j0 - loc0 : j0; };
  auto src_vec = [&](int s, int j0) {
    if constexpr (!CHUNK) return (N % 8) == 0 && j0 + KT <= N;  // tiles start at multiples of 64
    const int len = src_len(s), jr = src_rel(s, j0);
    return (len % 8) == 0 && (jr & 7) == 0 && jr >= 0 && jr + KT <= len;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const float sc = kLog2e / sqrtf((float)(D + DR));
  const int q_hi = nQT - 1 - pr;
  const int nq = (!paired || q_hi == pr) ? 1 : 2;

  for (int qn = 0; qn < nq; ++qn) {
    const int qt = qn == 0 ? q_hi : pr;
    if (qn > 0) __syncthreads();  // the LDS buffers are reused
    const int i0 = q0 + qt * QT, qw0 = i0 + 32 * wave;
    if (i0 >= N) continue;  // past a short sequence of a ragged batch (uniform per workgroup)
    const int qi = qw0 + lr;  // this lane's query
    const int i_last = min(i0 + QT - 1, N - 1);
    const int wi_last = min(qw0 + 31, N - 1);

    f16x8 qf[NQ];
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        u32x4 v = (qi < N) ? *(const u32x4*)(Qp + (size_t)(qi - q0) * D + 16 * st + 8 * lg) : z;
        qf[st] = __builtin_bit_cast(f16x8, v);
      }
#pragma unroll
      for (int st = D / 16; st < NQ; ++st) {
        u32x4 v = (qi < N) ? *(const u32x4*)(QRp + (size_t)qi * DR + 16 * (st - D / 16) + 8 * lg)
                           : z;
        qf[st] = __builtin_bit_cast(f16x8, v);
      }
    }
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_ref = kNegBig, l_run = 0.f;

    // Passes: for each key tile, the global source (if any pair of the
    // workgroup is at distance >= w) then the local source (if any is < w).
    const int j_end = min(N, i0 + QT);
    auto need_glob = [&](int j0) { return i_last - j0 >= w; };
    auto need_loc = [&](int j0) { return w > 0 && max(i0 - (j0 + KT - 1), 0) < w; };
    int j0 = 0, src = need_glob(0) ? 0 : 1;  // src 0 = global, 1 = local
    Stage<D, DR> stg;
    load_pass<D, DR>(stg, src ? Kl : Kg, src ? Vl : Vg, src_len(src), src_rel(src, j0),
                     src_vec(src, j0), KRb);
    store_pass<D, DR>(stg, sm.k[0], sm.v[0]);
    __syncthreads();
    int buf = 0;
    while (true) {
      int nj0 = j0, nsrc;
      if (src == 0 && need_loc(j0)) {
        nsrc = 1;
      } else {
        nj0 = j0 + KT;
        nsrc = need_glob(nj0) ? 0 : 1;
      }
      const bool has_next = nj0 < j_end;
      if constexpr (D == 64) {
        // V of the next pass is fetched now and stored after the first half;
        // K is fetched then and stored at the end (its LDS buffer is free
        // for the whole pass), so only one of the two is held in registers.
        if (has_next)
          load_v<D, DR>(stg.v, nsrc ? Vl : Vg, src_len(nsrc), src_rel(nsrc, nj0),
                        src_vec(nsrc, nj0));
      } else {
        if (has_next)
          load_pass<D, DR>(stg, nsrc ? Kl : Kg, nsrc ? Vl : Vg, src_len(nsrc), src_rel(nsrc, nj0),
                           src_vec(nsrc, nj0), KRb);
      }

      const WavePass wp = wave_pass_info(j0, src, qw0, wi_last, qi, lg, N, w);
      if constexpr (D == 64) {
        if (wp.part)
          wave_half<D, DR>(0, sm.k[buf], sm.v[buf], qf, o, m_ref, l_run, wp.masked, wp.keep_lo,
                           wp.keep_hi, sc, lr, lg);
        if (has_next) {
          store_v<D, DR>(stg.v, sm.v[buf ^ 1]);
          load_k<D, DR>(stg.k, nsrc ? Kl : Kg, src_len(nsrc), src_rel(nsrc, nj0), KRb);
        }
        if (wp.part)
          wave_half<D, DR>(1, sm.k[buf], sm.v[buf], qf, o, m_ref, l_run, wp.masked, wp.keep_lo,
                           wp.keep_hi, sc, lr, lg);
        if (!has_next) break;
        store_k<D, DR>(stg.k, sm.k[buf ^ 1]);
      } else {
        if (wp.part)
          wave_pass<D, DR>(sm.k[buf], sm.v[buf], qf, o, m_ref, l_run, wp.masked, wp.keep_lo,
                           wp.keep_hi, sc, lr, lg);
        if (!has_next) break;
        store_pass<D, DR>(stg, sm.k[buf ^ 1], sm.v[buf ^ 1]);
      }
      __syncthreads();
      buf ^= 1;
      j0 = nj0;
      src = nsrc;
    }

    if (qi < N) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const float inv = 1.f / l_tot;
      if (LSE && lg == 0)  // m_ref and l are in base 2
        p.lse[(size_t)bh * N + qi] = (m_ref + __log2f(l_tot)) * 0.6931471805599453f;
      // the row index and the lane's column offset are formed here (the empty
      // asm keeps the compiler from computing the 64-bit address before the
      // pass loop and holding it)
      int qr = qi - q0, dl = 4 * lg;
      __asm__ volatile("" : "+v"(qr), "+v"(dl));
      bf16* out = (bf16*)p.o + (orow0 + qr) * (size_t)(H * D) + (size_t)h * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + dl;
          u32x2 v;
          v[0] = pack_bf16x2(o[db][4 * rq + 0] * inv, o[db][4 * rq + 1] * inv);
          v[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
          *(u32x2*)(out + d) = v;
        }
    } else {
      (void)__shfl_xor(l_run, 32);  // keep the exchange wave-uniform
    }
  }
}

// ---------------------------------------------------------------------------
// d_k = 128 whole prefills with N a multiple of 64 (every key tile complete):
// eight waves of 32 queries (256 per workgroup, two waves per SIMD) share each
// key/value tile.  Tiles arrive by direct buffer loads into a four-stage LDS
// ring three passes ahead, so no staging registers, LDS stores or their
// address arithmetic are needed, and each tile is fetched once per 256
// queries.  The rows are unpadded, with an XOR chunk swizzle that keeps the
// fragment reads of 16 consecutive rows on distinct banks.  Per wave a pass is
// the one of attn_prefill_f16 (scores, keep mask and running maximum,
// exponentials, P.V).
constexpr int WQT = 256;  // queries per workgroup
constexpr int WNS = 4;    // stages of the LDS ring
constexpr int WD = 128;   // d_k

// DR = 64 (the decoupled-RoPE variant): the shared rotary keys of the tile's
// positions in a region of their own ([key][d_R], 128-byte rows swizzled as
// V^T's), since one buffer load reads one array.
template <int DR>
struct RingStage {
  f16 k[KT * WD];   // [key][d], chunk c of row r at slot c ^ (r & 15)
  f16 kr[KT * DR];  // [key][d_R], chunk c of row r at slot c ^ ((r >> 1) & 7)
  f16 v[WD * KT];   // [d][key], chunk c of row r at slot c ^ ((r >> 1) & 7)
};
template <>
struct RingStage<0> {
  f16 k[KT * WD];
  f16 v[WD * KT];
};
static_assert(sizeof(RingStage<0>) == 32768, "two 16 KB tiles");
static_assert(sizeof(RingStage<64>) == 40960, "16 + 8 + 16 KB");

__device__ __forceinline__ int wk_off(int row, int ch) { return row * WD + 8 * (ch ^ (row & 15)); }
__device__ __forceinline__ int wv_off(int row, int ch) {
  return row * KT + 8 * (ch ^ ((row >> 1) & 7));
}

// exp_and_pv on the ring's swizzled V^T tile.  Every V^T fragment of the pass
// is requested before the exponentials, so all of their LDS latency hides
// under them (1B-layer attention: 1.174 ms, against 1.192 with three of the
// four column blocks and 1.210-1.223 with two, in one run).
__device__ __forceinline__ void ring_exp_pv(const f16* sv, const f32x16 (&s)[2],
                                            f32x16 (&o)[WD / 32], float m_ref, float& l_run,
                                            float sc, int lr, int lg) {
  f16x8 vf[WD / 32][4];
#pragma unroll
  for (int db = 0; db < WD / 32; ++db)
#pragma unroll
    for (int u = 0; u < 4; ++u) vf[db][u] = *(const f16x8*)(sv + wv_off(32 * db + lr, lg + 2 * u));
  f16x8 pf[4];
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 one2 = {(f16)1.f, (f16)1.f};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int c = 0; c < 8; c += 2) {
      const float e0 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + c], sc, -m_ref));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(s[u >> 1][8 * (u & 1) + c + 1], sc, -m_ref));
      const h2 ph = __builtin_bit_cast(h2, pack_f16x2(e0, e1));
      l_run = __builtin_amdgcn_fdot2(ph, one2, l_run, false);
      pf[u][c] = ph[0];
      pf[u][c + 1] = ph[1];
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int db = 0; db < WD / 32; ++db) o[db] = mfma32x32x16(vf[db][u], pf[u], o[db]);
}

// LSE: also store each query's log-sum-exp in p.lse.  DR = 64: the
// decoupled-RoPE variant (whole prefill; three stages fit in LDS).
template <bool LSE, int DR = 0>
__global__ __launch_bounds__(512, 1) void attn_prefill_ring(PrefillProblem p, int nQT, int nPair,
                                                            int remap) {
  static_assert(DR == 0 || !LSE, "the variant's prefill stores no log-sum-exp");
  constexpr int NS = DR > 0 ? 3 : WNS;  // stages
  constexpr int LPP = DR > 0 ? 5 : 4;   // loads per lane and pass
  constexpr int NQ = (WD + DR) / 16;    // 16-wide steps of the score contraction
  __shared__ RingStage<DR> sm[NS];
  const int H = p.H, BH = p.B * p.H, w = p.w;
  int pr, bh;
  {
    const int bid = blockIdx.x;
    if (remap) {  // every tile of one (batch, head) on one XCD
      const int x = bid % kNumXcd, k = bid / kNumXcd;
      pr = k % nPair;
      bh = (k / nPair) * kNumXcd + x;
    } else {
      pr = bid / BH;
      bh = bid % BH;
    }
  }
  const int b = bh / H, h = bh % H;
  // Chunk form: the queries are positions q0 .. N-1 (Q and o hold N - q0
  // rows), the local arrays hold positions loc0 .. N-1 (loc0 a multiple of
  // the key tile), the global arrays 0 .. N-1.  A whole prefill has
  // q0 = loc0 = 0.
  const int N = p.N, q0 = p.q0, loc0 = p.loc0;
  const int nqr = N - q0, nloc = N - loc0;
  const size_t slice = (size_t)bh * N * WD, lslice = (size_t)bh * nloc * WD;
  const f16* Qp = (const f16*)p.Q + (size_t)bh * nqr * WD;
  const size_t orow0 = (size_t)b * nqr;
  const int bytes = N * WD * 2, lbytes = nloc * WD * 2;  // < 2 GiB (checked by the launcher)
  // (four scalars, not arrays: an array indexed by the source would be
  // placed in memory)
  const __amdgpu_buffer_rsrc_t rKg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const f16*)p.K_glob + slice), (short)0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rKl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const f16*)p.K_loc + lslice), (short)0, lbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rVg = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const f16*)p.V_glob + slice), (short)0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rVl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const f16*)p.V_loc + lslice), (short)0, lbytes, 0x00020000);
  // rotary keys of sequence b (positions 0 .. N-1, every head) and queries
  const __amdgpu_buffer_rsrc_t rKR = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(DR > 0 ? (const f16*)p.KR + (size_t)b * N * DR : (const f16*)p.Q), (short)0,
      N * DR * 2, 0x00020000);
  const f16* QRp = DR > 0 ? (const f16*)p.QR + (size_t)bh * nqr * DR : nullptr;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const float sc = kLog2e / sqrtf((float)(WD + DR));
  // This lane's fixed byte offsets within a tile: LDS slot P = (8 i + wave) 64
  // + lane of the K tile (row P / 16, slot P % 16) and of the V^T tile (row
  // P / 8, slot P % 8), loaded from the chunk the swizzle puts there.
  unsigned vk[2], vv[2], vl[2];  // V^T rows: N (global) or nloc (local) keys apart
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = (8 * i + wave) * 64 + lane;
    const int kr = P >> 4, kc = (P & 15) ^ (kr & 15);
    vk[i] = (unsigned)((kr * WD + 8 * kc) * 2);
    const int vr = P >> 3, vc = (P & 7) ^ ((vr >> 1) & 7);
    vv[i] = (unsigned)((vr * N + 8 * vc) * 2);
    vl[i] = (unsigned)((vr * nloc + 8 * vc) * 2);
  }
  // rotary region: slot P = wave 64 + lane (row P / 8, slot P % 8)
  unsigned vkr = 0;
  if constexpr (DR > 0) {
    const int P = wave * 64 + lane, rr = P >> 3, rc = (P & 7) ^ ((rr >> 1) & 7);
    vkr = (unsigned)((rr * DR + 8 * rc) * 2);
  }
  auto issue = [&](int j0, int src, int stg) {
    const int jr = src ? j0 - loc0 : j0;  // first row of the tile in its source's arrays
    if constexpr (DR > 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rKR, (__attribute__((address_space(3))) void*)(sm[stg].kr + wave * 512), 16, vkr,
          j0 * DR * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src ? rKl : rKg, (__attribute__((address_space(3))) void*)(sm[stg].k + (8 * i + wave) * 512), 16,
          vk[i], jr * WD * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src ? rVl : rVg, (__attribute__((address_space(3))) void*)(sm[stg].v + (8 * i + wave) * 512), 16,
          src ? vl[i] : vv[i], jr * 2, 0, 0);
  };
  // s_waitcnt vmcnt(LPP n) (lgkmcnt and expcnt left alone): at most n later
  // passes in flight; N's low 4 bits in [3:0], its high 2 bits in [15:14]
  constexpr int W1 = ((LPP >> 4) << 14) | 0x0F70 | (LPP & 15);
  constexpr int W2 = (((2 * LPP) >> 4) << 14) | 0x0F70 | ((2 * LPP) & 15);
  auto wait_passes = [](int n) {
    if (n >= 2)
      __builtin_amdgcn_s_waitcnt(W2);
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt(W1);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  const int q_hi = nQT - 1 - pr;
  const int nq = q_hi == pr ? 1 : 2;
  for (int qn = 0; qn < nq; ++qn) {
    const int qt = qn == 0 ? q_hi : pr;
    if (qn > 0) __syncthreads();  // every wave is done with the ring
    const int i0 = q0 + qt * WQT, qw0 = i0 + 32 * wave, qi = qw0 + lr;
    const int i_last = min(i0 + WQT - 1, N - 1), wi_last = min(qw0 + 31, N - 1);
    f16x8 qf[NQ];
    {
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int st = 0; st < WD / 16; ++st) {
        const u32x4 v =
            qi < N ? *(const u32x4*)(Qp + (size_t)(qi - q0) * WD + 16 * st + 8 * lg) : z;
        qf[st] = __builtin_bit_cast(f16x8, v);
      }
#pragma unroll
      for (int st = WD / 16; st < NQ; ++st) {
        const u32x4 v = qi < N ? *(const u32x4*)(QRp + (size_t)(qi - q0) * DR +
                                                 16 * (st - WD / 16) + 8 * lg)
                               : z;
        qf[st] = __builtin_bit_cast(f16x8, v);
      }
    }
    f32x16 o[WD / 32];
#pragma unroll
    for (int db = 0; db < WD / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
    float m_ref = kNegBig, l_run = 0.f;

    const int j_end = min(N, i0 + WQT);
    auto need_glob = [&](int j0) { return i_last - j0 >= w; };
    auto need_loc = [&](int j0) { return w > 0 && max(i0 - (j0 + KT - 1), 0) < w; };
    auto next = [&](int& j0, int& src) {
      if (src == 0 && need_loc(j0)) {
        src = 1;
      } else {
        j0 += KT;
        src = need_glob(j0) ? 0 : 1;
      }
    };
    int cj = 0, cs = need_glob(0) ? 0 : 1;  // the pass computed now
    int aj = cj, as = cs;                   // the next pass to load
    int issued = 0;
#pragma unroll
    for (int k = 0; k < NS - 1; ++k)
      if (aj < j_end) {
        issue(aj, as, k);
        next(aj, as);
        ++issued;
      }
    for (int t = 0; cj < j_end; ++t) {
      wait_passes(issued - t - 1);  // this lane's loads of pass t have landed
      lds_barrier();                // everyone's have; everyone is done with pass t-1
      if (aj < j_end) {
        issue(aj, as, (t + NS - 1) % NS);
        next(aj, as);
        ++issued;
      }
      const RingStage<DR>& S = sm[t % NS];
      const WavePass wp = wave_pass_info(cj, cs, qw0, wi_last, qi, lg, N, w);
      if (wp.part) {
        f16x8 kf[2][NQ];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = 32 * kb + key_perm(lr);
#pragma unroll
          for (int st = 0; st < WD / 16; ++st)
            kf[kb][st] = *(const f16x8*)(S.k + wk_off(row, 2 * st + lg));
          if constexpr (DR > 0) {
#pragma unroll
            for (int st = WD / 16; st < NQ; ++st)
              kf[kb][st] = *(const f16x8*)(S.kr + row * DR +
                                           8 * ((2 * (st - WD / 16) + lg) ^ ((row >> 1) & 7)));
          }
        }
        f32x16 s[2];
        mfma_scores<WD, DR>(kf, qf, s);
        mask_and_max<WD>(s, o, m_ref, l_run, wp.masked, wp.keep_lo, wp.keep_hi, sc);
        ring_exp_pv(S.v, s, o, m_ref, l_run, sc, lr, lg);
      }
      next(cj, cs);
    }

    if (qi < N) {
      const float l_tot = l_run + __shfl_xor(l_run, 32);
      const float inv = 1.f / l_tot;
      if (LSE && lg == 0)  // m_ref and l are in base 2
        p.lse[(size_t)bh * N + qi] = (m_ref + __log2f(l_tot)) * 0.6931471805599453f;
      bf16* out = (bf16*)p.o + (orow0 + (qi - q0)) * (size_t)(H * WD) + (size_t)h * WD;
#pragma unroll
      for (int db = 0; db < WD / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d = 32 * db + 8 * rq + 4 * lg;
          u32x2 v;
          v[0] = pack_bf16x2(o[db][4 * rq + 0] * inv, o[db][4 * rq + 1] * inv);
          v[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
          *(u32x2*)(out + d) = v;
        }
    } else {
      (void)__shfl_xor(l_run, 32);  // keep the exchange wave-uniform
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: 64 queries per workgroup, four lanes per query (lane part
// `pt` owns dims pt, pt+4, ...), keys staged 32 at a time.
constexpr int FQ = 64, FK = 32;

template <int D>
__global__ __launch_bounds__(256) void attn_prefill_f32(PrefillProblem p) {
  __shared__ float sk[2][FK][D];
  __shared__ float sv[2][FK][D];
  const int N = p.N, H = p.H, w = p.w;
  const int nQT = (N + FQ - 1) / FQ;
  const int qt = nQT - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t off = ((size_t)b * H + h) * N * D;
  const float* Qp = (const float*)p.Q + off;
  const float* Ks[2] = {(const float*)p.K_loc + off, (const float*)p.K_glob + off};
  const float* Vs[2] = {(const float*)p.V_loc + off, (const float*)p.V_glob + off};
  const int tid = threadIdx.x, qi = qt * FQ + tid / 4, pt = tid & 3;
  constexpr int E = D / 4;
  float q[E], acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = (qi < N) ? Qp[(size_t)qi * D + pt + 4 * e] : 0.f;
    acc[e] = 0.f;
  }
  const float scale = 1.f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  const int j_end = min(N, qt * FQ + FQ);
  for (int j0 = 0; j0 < j_end; j0 += FK) {
    __syncthreads();
    for (int e = tid; e < FK * D; e += 256) {
      const int kk = e / D, d = e % D, j = j0 + kk;
#pragma unroll
      for (int src = 0; src < 2; ++src) sk[src][kk][d] = (j < N) ? Ks[src][(size_t)j * D + d] : 0.f;
    }
    for (int e = tid; e < FK * D; e += 256) {
      const int d = e / FK, kk = e % FK, j = j0 + kk;
#pragma unroll
      for (int src = 0; src < 2; ++src) sv[src][kk][d] = (j < N) ? Vs[src][(size_t)d * N + j] : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < FK; ++kk) {
      const int j = j0 + kk;
      const int src = (qi - j < w) ? 0 : 1;  // Eq. (3): i - j < w -> full state
      const float* kr = sk[src][kk];
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot = fmaf(q[e], kr[pt + 4 * e], dot);
      dot += __shfl_xor(dot, 1);
      dot += __shfl_xor(dot, 2);
      if (j > qi || j >= N) continue;
      const float sj = dot * scale;
      const float m_new = fmaxf(m, sj);
      const float corr = expf(m - m_new), pj = expf(sj - m_new);
      l = l * corr + pj;
      const float* vr = sv[src][kk];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pj, vr[pt + 4 * e], acc[e] * corr);
      m = m_new;
    }
  }
  if (qi >= N) return;
  if (p.lse != nullptr && pt == 0) p.lse[((size_t)b * H + h) * N + qi] = m + logf(l);
  float* out = (float*)p.o + ((size_t)b * N + qi) * (size_t)(H * D) + (size_t)h * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) out[pt + 4 * e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_attn_prefill(const PrefillProblem& p_in, dar_dtype dt, hipStream_t s) {
  // Distances never exceed N - 1, so any w >= N selects the local path for
  // every pair; clamping keeps the kernels' distance arithmetic in range.
  PrefillProblem p = p_in;
  if (p.w > p.N) p.w = p.N;
  const int BH = p.B * p.H;
  if (dt == DAR_BF16) {
    const int nQT = (p.N - p.q0 + QT - 1) / QT;
    // d_k = 64 fits three waves per SIMD, so one tile per workgroup (longest
    // first) keeps more of them resident; at d_k = 128 (two per SIMD) pairing
    // balances the workgroups instead.
    const int paired = p.d_k == 128 ? 1 : 0;
    const int nPair = paired ? (nQT + 1) / 2 : nQT;
    const int remap = (BH % kNumXcd) == 0 ? 1 : 0;
    const dim3 grid(nPair * BH);
    const bool chunk = p.q0 != 0 || p.loc0 != 0;
#define DAR_ATTN(DV, CV, LV) \
  hipLaunchKernelGGL((attn_prefill_f16<DV, CV, LV>), grid, dim3(256), 0, s, p, nQT, nPair, remap, \
                     paired)
    if (chunk && p.lse != nullptr) return hipErrorInvalidValue;
    const bool lse = p.lse != nullptr;
    if (p.cu != nullptr && (chunk || lse || p.d_R > 0 || p.T < 1)) return hipErrorInvalidValue;
    if (p.d_R > 0) {  // decoupled-RoPE variant: whole prefill, d_R = 64
      if (chunk || lse || p.d_R != 64) return hipErrorInvalidValue;
      if (p.d_k == 128 && p.N % KT == 0 && (long)p.N * WD * 2 < 0x7fffffffL) {
        const int nQW = (p.N + WQT - 1) / WQT, nPW = (nQW + 1) / 2;
        hipLaunchKernelGGL((attn_prefill_ring<false, 64>), dim3(nPW * BH), dim3(512), 0, s, p, nQW,
                           nPW, remap);
        return hipGetLastError();
      }
      if (p.d_k == 64)
        hipLaunchKernelGGL((attn_prefill_f16<64, false, false, 64>), grid, dim3(256), 0, s, p, nQT,
                           nPair, remap, paired);
      else
        hipLaunchKernelGGL((attn_prefill_f16<128, false, false, 64>), grid, dim3(256), 0, s, p,
                           nQT, nPair, remap, paired);
      return hipGetLastError();
    }
    if (p.d_k == 128 && p.cu == nullptr && p.N % KT == 0 && p.loc0 % KT == 0 &&
        (long)p.N * WD * 2 < 0x7fffffffL) {
      // complete key tiles (a whole prefill, or a chunk whose local arrays
      // start on a tile): the ring kernel (pairs of query tiles)
      const int nQW = (p.N - p.q0 + WQT - 1) / WQT, nPW = (nQW + 1) / 2;
      if (lse)
        hipLaunchKernelGGL(attn_prefill_ring<true>, dim3(nPW * BH), dim3(512), 0, s, p, nQW, nPW,
                           remap);
      else
        hipLaunchKernelGGL(attn_prefill_ring<false>, dim3(nPW * BH), dim3(512), 0, s, p, nQW, nPW,
                           remap);
      return hipGetLastError();
    }
    if (p.d_k == 64) {
      if (chunk) DAR_ATTN(64, true, false);
      else if (lse) DAR_ATTN(64, false, true);
      else DAR_ATTN(64, false, false);
    } else {
      if (chunk) DAR_ATTN(128, true, false);
      else if (lse) DAR_ATTN(128, false, true);
      else DAR_ATTN(128, false, false);
    }
#undef DAR_ATTN
  } else {
    if (p.cu != nullptr) return hipErrorInvalidValue;  // ragged batches: bf16 mode
    const dim3 grid((p.N + FQ - 1) / FQ, p.H, p.B);
    if (p.d_k == 64)
      hipLaunchKernelGGL(attn_prefill_f32<64>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_prefill_f32<128>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace dar
