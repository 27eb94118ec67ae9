// Backward of the fused dual-source causal attention (prefill).
//
// "Dual Dimensionality for Local and Global Attention", Eqs. (3)-(4) and the
// training remark after Eq. (4): query i attends to every key j <= i through
// the full-state key/value (K_loc, V_loc) when i - j < w and through the
// bottleneck one (K_glob, V_glob) otherwise, so the gradient of each pair
// flows to the source that pair used; the bottleneck weights learn only from
// global pairs.  With s_ij = q_i . k_j / sqrt(d_k), p_ij = softmax_j(s_ij),
// lse_i = log sum_j exp(s_ij), dp_ij = dO_i . v_j and
// D_i = sum_j p_ij dp_ij = dO_i . o_i:
//   ds_ij = p_ij (dp_ij - D_i)
//   dq_i  = sum_j ds_ij k_j / sqrt(d_k)
//   dk_j  = sum_i ds_ij q_i / sqrt(d_k)     (into the source of pair (i, j))
//   dv_j  = sum_i p_ij dO_i                 (likewise)
//
// bf16 mode runs the MFMA kernels further below (bwd_dq_mfma, and bwd_dkv_mfma
// at d_k 64 or bwd_dkv_split at d_k 128).
// fp32 mode runs two VALU kernels in fp32 (the gradients are fp32 in both
// modes):
//   bwd_dq:  64 queries per workgroup, four lanes per query (lane part pt owns
//            dims pt, pt + 4, ...).  Keys of both sources are staged 32 at a
//            time.  lse_i comes from the forward or from a first sweep (online
//            maximum and sum); D_i and lse_i are stored for the second kernel
//            and a second sweep accumulates dq_i.
//   bwd_dkv: d_k / 16 lanes per key (16 dims each), 64 or 32 keys per
//            workgroup, both sources' k, v and gradient accumulators in
//            registers.  Queries i >= j stream through LDS 32 at a time with
//            their dO, lse and D; each pair updates the accumulators of its
//            source.
// The pair selection is taken per pair, as Eq. (3) writes it.
#include <math.h>

#include <type_traits>

#include "dar_common.hpp"

namespace dar {

namespace {

constexpr int BQ = 64;   // queries per bwd_dq workgroup
constexpr int BK = 32;   // keys per staged tile (bwd_dq)
constexpr int BQ2 = 32;  // queries per staged tile (bwd_dkv)

// Sum over the LP consecutive lanes that share one row.
template <int LP>
__device__ __forceinline__ float row_sum(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  if constexpr (LP == 8) v += __shfl_xor(v, 4);
  return v;
}

template <bool BF, int D>
__global__ __launch_bounds__(256) void bwd_dq(BwdProblem p) {
  typedef typename std::conditional<BF, f16, float>::type TQ;  // Q, K, V
  typedef typename std::conditional<BF, bf16, float>::type TO;  // o, dO
  constexpr int LP = 4, E = D / LP;
  __shared__ float sk[2][BK][D];  // [source: 0 local, 1 global][key][dim]
  __shared__ float sv[2][BK][D];
  const int N = p.N, H = p.H, w = p.w, BH = p.B * p.H;
  const int nQT = (N + BQ - 1) / BQ;
  const int qt = nQT - 1 - (int)(blockIdx.x / BH);  // longest query tiles first
  const int bh = (int)(blockIdx.x % BH), b = bh / H, h = bh % H;
  const TQ* Qp = (const TQ*)p.Q + (size_t)bh * N * D;
  const TQ* Ks[2] = {(const TQ*)p.K_loc + (size_t)bh * N * D,
                     (const TQ*)p.K_glob + (size_t)bh * N * D};
  const TQ* Vs[2] = {(const TQ*)p.V_loc + (size_t)bh * D * N,   // [d][n]
                     (const TQ*)p.V_glob + (size_t)bh * D * N};
  const int tid = threadIdx.x, pt = tid & (LP - 1);
  const int qi = qt * BQ + tid / LP;
  const bool qv = qi < N;
  const int qc = qv ? qi : N - 1;  // a valid row for the loads of idle lanes
  const size_t orow = ((size_t)b * N + qc) * (size_t)(H * D) + (size_t)h * D;
  float q[E], g[E], acc[E];
  float Dd = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = pt + LP * e;
    q[e] = to_f32(Qp[(size_t)qc * D + t]);
    g[e] = to_f32(((const TO*)p.dO)[orow + t]);
    Dd = fmaf(g[e], to_f32(((const TO*)p.o)[orow + t]), Dd);
    acc[e] = 0.f;
  }
  Dd = row_sum<LP>(Dd);
  const float sc = 1.f / sqrtf((float)D);
  const int i_last = min(N, qt * BQ + BQ) - 1;

  // lse_i: the forward's, or sweep 1 over j <= i
  float m = -INFINITY, l = 0.f;
  if (p.lse_in != nullptr) {
    m = p.lse_in[(size_t)bh * N + qc];
    l = 1.f;
  }
  for (int j0 = 0; p.lse_in == nullptr && j0 <= i_last; j0 += BK) {
    __syncthreads();
    for (int e = tid; e < BK * D; e += 256) {
      const int kk = e / D, d = e % D, j = j0 + kk;
#pragma unroll
      for (int s = 0; s < 2; ++s) sk[s][kk][d] = j < N ? to_f32(Ks[s][(size_t)j * D + d]) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < BK; ++kk) {
      const int j = j0 + kk;
      const float* kr = sk[(qi - j < w) ? 0 : 1][kk];  // Eq. (3)
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot = fmaf(q[e], kr[pt + LP * e], dot);
      dot = row_sum<LP>(dot);
      if (j <= qi && qv) {
        const float s = dot * sc, m_new = fmaxf(m, s);
        l = l * expf(m - m_new) + expf(s - m_new);
        m = m_new;
      }
    }
  }
  const float lse = m + logf(l);
  if (qv && pt == 0) {
    p.lse[(size_t)bh * N + qi] = lse;
    p.Dd[(size_t)bh * N + qi] = Dd;
  }

  // sweep 2: dq_i = sum_j p_ij (dp_ij - D_i) k_j / sqrt(d_k)
  for (int j0 = 0; j0 <= i_last; j0 += BK) {
    __syncthreads();
    for (int e = tid; e < BK * D; e += 256) {
      const int kk = e / D, d = e % D, j = j0 + kk;
#pragma unroll
      for (int s = 0; s < 2; ++s) sk[s][kk][d] = j < N ? to_f32(Ks[s][(size_t)j * D + d]) : 0.f;
    }
    for (int e = tid; e < BK * D; e += 256) {
      const int d = e / BK, kk = e % BK, j = j0 + kk;
#pragma unroll
      for (int s = 0; s < 2; ++s) sv[s][kk][d] = j < N ? to_f32(Vs[s][(size_t)d * N + j]) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < BK; ++kk) {
      const int j = j0 + kk;
      const int src = (qi - j < w) ? 0 : 1;  // Eq. (3)
      const float* kr = sk[src][kk];
      const float* vr = sv[src][kk];
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s = fmaf(q[e], kr[pt + LP * e], s);
        dp = fmaf(g[e], vr[pt + LP * e], dp);
      }
      s = row_sum<LP>(s);
      dp = row_sum<LP>(dp);
      const float pr = (j <= qi && qv) ? expf(s * sc - lse) : 0.f;
      const float ds = pr * (dp - Dd) * sc;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kr[pt + LP * e], acc[e]);
    }
  }
  if (qv) {
    float* dq = p.dQ + ((size_t)bh * N + qi) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) dq[pt + LP * e] = acc[e];
  }
}

template <bool BF, int D>
__global__ __launch_bounds__(256) void bwd_dkv(BwdProblem p) {
  typedef typename std::conditional<BF, f16, float>::type TQ;
  typedef typename std::conditional<BF, bf16, float>::type TO;
  constexpr int LP = D / 16, E = 16, BKV = 256 / LP;  // keys per workgroup
  __shared__ float sq[BQ2][D];
  __shared__ float sg[BQ2][D];
  __shared__ float sl[BQ2], sd[BQ2];
  const int N = p.N, H = p.H, w = p.w, BH = p.B * p.H;
  const int kt = (int)(blockIdx.x / BH);  // small key tiles (most queries) first
  const int bh = (int)(blockIdx.x % BH), b = bh / H, h = bh % H;
  const int tid = threadIdx.x, pt = tid % LP;
  const int j = kt * BKV + tid / LP;
  const bool jv = j < N;
  const int jc = jv ? j : N - 1;
  const TQ* Qp = (const TQ*)p.Q + (size_t)bh * N * D;
  const size_t koff = (size_t)bh * N * D + (size_t)jc * D;
  float kL[E], kG[E], vL[E], vG[E], dkL[E], dkG[E], dvL[E], dvG[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = pt + LP * e;
    kL[e] = to_f32(((const TQ*)p.K_loc)[koff + t]);
    kG[e] = to_f32(((const TQ*)p.K_glob)[koff + t]);
    vL[e] = to_f32(((const TQ*)p.V_loc)[((size_t)bh * D + t) * N + jc]);
    vG[e] = to_f32(((const TQ*)p.V_glob)[((size_t)bh * D + t) * N + jc]);
    dkL[e] = dkG[e] = dvL[e] = dvG[e] = 0.f;
  }
  const float sc = 1.f / sqrtf((float)D);
  for (int i0 = kt * BKV; i0 < N; i0 += BQ2) {
    __syncthreads();
    for (int e = tid; e < BQ2 * D; e += 256) {
      const int ii = e / D, d = e % D, i = i0 + ii;
      const bool iv = i < N;
      sq[ii][d] = iv ? to_f32(Qp[(size_t)i * D + d]) : 0.f;
      sg[ii][d] = iv ? to_f32(((const TO*)p.dO)[((size_t)b * N + i) * (size_t)(H * D) +
                                                (size_t)h * D + d])
                     : 0.f;
    }
    if (tid < BQ2) {
      const int i = i0 + tid;
      sl[tid] = i < N ? p.lse[(size_t)bh * N + i] : 0.f;
      sd[tid] = i < N ? p.Dd[(size_t)bh * N + i] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < BQ2; ++ii) {
      const int i = i0 + ii;
      const bool keep = jv && i >= j && i < N;
      const float* qr = sq[ii];
      const float* gr = sg[ii];
      if (i - j < w) {  // Eq. (3): full-state key/value
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s = fmaf(qr[pt + LP * e], kL[e], s);
          dp = fmaf(gr[pt + LP * e], vL[e], dp);
        }
        s = row_sum<LP>(s);
        dp = row_sum<LP>(dp);
        const float pr = keep ? expf(s * sc - sl[ii]) : 0.f;
        const float ds = pr * (dp - sd[ii]) * sc;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dvL[e] = fmaf(pr, gr[pt + LP * e], dvL[e]);
          dkL[e] = fmaf(ds, qr[pt + LP * e], dkL[e]);
        }
      } else {  // bottleneck key/value
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s = fmaf(qr[pt + LP * e], kG[e], s);
          dp = fmaf(gr[pt + LP * e], vG[e], dp);
        }
        s = row_sum<LP>(s);
        dp = row_sum<LP>(dp);
        const float pr = keep ? expf(s * sc - sl[ii]) : 0.f;
        const float ds = pr * (dp - sd[ii]) * sc;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dvG[e] = fmaf(pr, gr[pt + LP * e], dvG[e]);
          dkG[e] = fmaf(ds, qr[pt + LP * e], dkG[e]);
        }
      }
    }
  }
  if (jv) {
    const size_t off = ((size_t)bh * N + j) * D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int t = pt + LP * e;
      p.dK_loc[off + t] = dkL[e];
      p.dK_glob[off + t] = dkG[e];
      p.dV_loc[off + t] = dvL[e];
      p.dV_glob[off + t] = dvG[e];
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernels (bf16 mode, fp16 Q/K/V).  32x32x16 fp16 MFMAs with fp32
// accumulation; softmax in base 2 (lse2_i = log2 sum_j 2^(s_ij log2(e)/sqrt(d_k))).
// Operand layout of mfma32x32x16: lane l gives row / column l % 32 and
// contraction elements 8 (l / 32) .. +8 of each 16-wide step; result
// register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
// Feeding the rows of the first product in the order row_perm (bits 2 and 3
// of the row index swapped) makes result registers 8u .. 8u+7 of lane l the
// rows 16u + 8 (l / 32) .. +8: exactly the B operand of a later product that
// contracts over those rows.
constexpr int MQ = 128;  // queries (bwd_dq_mfma) or keys (bwd_dkv_mfma) per workgroup
constexpr int MB = 32;   // keys or queries per staged block

__device__ __forceinline__ int row_perm(int r) {  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Row offset (within a 32-row block fed through row_perm) of result register r.
__device__ __forceinline__ constexpr int perm_row(int r, int lg) {
  return 16 * (r >> 3) + 8 * lg + (r & 7);
}

// Pair classification of a 32 x 32 block for one source, from the distance
// range of its pairs: any kept pair, and whether the element mask is needed.
// Kept pairs: local 0 <= i - j < w, global i - j >= w, with i, j < N.
struct BlockPass {
  bool part, masked;
};
__device__ __forceinline__ BlockPass block_pass(int src, int q0, int k0, int N, int w) {
  const int q_last = min(q0 + 31, N - 1), k_last = min(k0 + 31, N - 1);
  const int dmax = q_last - k0, dmin = q0 - k_last;
  BlockPass r{false, false};
  if (q0 >= N || k0 >= N || dmax < 0) return r;
  if (src == 0) {
    r.part = w > 0 && max(dmin, 0) < w;
    r.masked = dmin < 0 || dmax >= w;
  } else {
    r.part = dmax >= w;
    r.masked = dmin < w;
  }
  r.masked = r.masked || q0 + 32 > N || k0 + 32 > N;
  return r;
}

__device__ __forceinline__ bool keep_pair(int src, int dist, int w) {
  return src == 0 ? (unsigned)dist < (unsigned)w : dist >= w;
}

// A 32-row block of a [n][D] fp16 array held in registers on its way to LDS:
// chunk c = tid + 256 i is row c / (D/8), columns 8 (c % (D/8)) .. +8.
template <int D>
struct Rows {
  static constexpr int NCH = MB * D / 8 / 256;
  u32x4 v[NCH];
};

// Rows r0 .. r0+31 of a row-major fp16 [n][D] array (zero past N).
template <int D>
__device__ __forceinline__ void load_rows(Rows<D>& x, const f16* src, int r0, int N) {
#pragma unroll
  for (int i = 0; i < Rows<D>::NCH; ++i) {
    const int c = threadIdx.x + 256 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
    x.v[i] = u32x4{0u, 0u, 0u, 0u};
    if (r0 + row < N) x.v[i] = *(const u32x4*)(src + (size_t)(r0 + row) * D + col);
  }
}

// ... stored as rows of pitch RP.
template <int D, int RP>
__device__ __forceinline__ void store_rows(const Rows<D>& x, f16* rows) {
#pragma unroll
  for (int i = 0; i < Rows<D>::NCH; ++i) {
    const int c = threadIdx.x + 256 * i, row = c / (D / 8), col = (c % (D / 8)) * 8;
    *(u32x4*)(rows + row * RP + col) = x.v[i];
  }
}

// Paired staging for the blocks that LDS also needs transposed: 128 threads
// (pi = 0 .. 127) each take two adjacent rows (or dims) of one 8-wide chunk,
// so the transposed copy is written as 4-byte pairs.  For a block of ROWS rows,
// pair slot q = pi + 128 i covers rows 2 (q % (ROWS/2)), +1 and columns
// 8 (q / (ROWS/2)) .. +8 (a wave's 4-byte writes then spread over the banks).
template <int D, int ROWS>
struct Pairs {
  static constexpr int NP = ROWS * D / 16 / 128;
  u32x4 a[NP], b[NP];  // the two rows
};

__device__ __forceinline__ uint32_t pack2(f16 lo, f16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// 16 bytes at row r, column col of a row-major array of 2-byte elements with
// n rows of stride ld; rows r >= n read as zeros.  BUF (the launcher's choice
// when every staged array is under 2 GiB): through a buffer resource, whose
// range check supplies the zeros without a branch; else a guarded load.
template <bool BUF>
__device__ __forceinline__ u32x4 load_row16(const void* base, int n, size_t ld, int r, int col) {
  if constexpr (BUF) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(n * ld * 2), 0x00020000);
    const unsigned off = ((unsigned)r * (unsigned)ld + (unsigned)col) * 2u;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return r < n ? *(const u32x4*)((const uint16_t*)base + (size_t)r * ld + col) : z;
  }
}

// Rows r0 .. r0+ROWS-1, columns 0 .. D-1 of a row-major fp16 array of row
// stride LDF (zero past N); with
// grad_ld > 0 the source is bf16 dO rows of stride grad_ld, held as bf16 bits
// (store_pairs<..., true> turns them into fp16), so that no instruction uses
// the loaded registers before the store and the loads stay in flight.
template <int D, int ROWS, bool BUF, int LDF = D>
__device__ __forceinline__ void load_pairs(Pairs<D, ROWS>& x, const void* src, size_t grad_ld,
                                           int r0, int N, int pi) {
  const size_t ld = grad_ld == 0 ? (size_t)LDF : grad_ld;
#pragma unroll
  for (int i = 0; i < Pairs<D, ROWS>::NP; ++i) {
    const int q = pi + 128 * i, row = 2 * (q % (ROWS / 2)), col = (q / (ROWS / 2)) * 8;
    x.a[i] = load_row16<BUF>(src, N, ld, r0 + row, col);
    x.b[i] = load_row16<BUF>(src, N, ld, r0 + row + 1, col);
  }
}

// ... as rows of pitch RP and transposed as [d][row] of pitch TP (BF: the
// registers hold bf16 bits, converted to fp16 here).  GP: extra halves after
// every 16 transposed rows (see DqSmem).
template <int D, int ROWS, int RP, int TP, bool BF = false, int GP = 0>
__device__ __forceinline__ void store_pairs(const Pairs<D, ROWS>& x, f16* rows, f16* cols,
                                            int pi) {
#pragma unroll
  for (int i = 0; i < Pairs<D, ROWS>::NP; ++i) {
    const int q = pi + 128 * i, row = 2 * (q % (ROWS / 2)), col = (q / (ROWS / 2)) * 8;
    const u32x4 va = BF ? bf16x8_to_f16x8(x.a[i]) : x.a[i];
    const u32x4 vb = BF ? bf16x8_to_f16x8(x.b[i]) : x.b[i];
    *(u32x4*)(rows + row * RP + col) = va;
    *(u32x4*)(rows + (row + 1) * RP + col) = vb;
    const f16x8 ha = __builtin_bit_cast(f16x8, va), hb = __builtin_bit_cast(f16x8, vb);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(uint32_t*)(cols + (col + e) * TP + GP * ((col + e) >> 4) + row) = pack2(ha[e], hb[e]);
  }
}

// Keys j0 .. j0+31 of V^T [D][n] (zero past N): pair slot q covers dims
// 2 (q / 4), +1 and keys 8 (q % 4) .. +8; stored as rows [key][d].
template <int D>
__device__ __forceinline__ void load_vt_pairs(Pairs<D, MB>& x, const f16* src, int j0, int N,
                                              int pi) {
#pragma unroll
  for (int i = 0; i < Pairs<D, MB>::NP; ++i) {
    const int q = pi + 128 * i, d = 2 * (q / (MB / 8)), kc = (q % (MB / 8)) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f16* p = src + (size_t)(d + h) * N + j0 + kc;
      u32x4 v;
      if ((N & 7) == 0 && j0 + kc + 8 <= N) {
        v = *(const u32x4*)p;
      } else {
        f16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = j0 + kc + e < N ? p[e] : (f16)0.f;
        v = __builtin_bit_cast(u32x4, t);
      }
      (h ? x.b[i] : x.a[i]) = v;
    }
  }
}

template <int D, int RP, int GP = 0>
__device__ __forceinline__ void store_vt_pairs(const Pairs<D, MB>& x, f16* rows, int pi) {
#pragma unroll
  for (int i = 0; i < Pairs<D, MB>::NP; ++i) {
    const int q = pi + 128 * i, d = 2 * (q / (MB / 8)), kc = (q % (MB / 8)) * 8;
    const f16x8 ha = __builtin_bit_cast(f16x8, x.a[i]), hb = __builtin_bit_cast(f16x8, x.b[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *(uint32_t*)(rows + (kc + e) * RP + GP * ((kc + e) >> 4) + d) = pack2(ha[e], hb[e]);
  }
}

// kt and v take 4-byte pair writes whose 64 lanes fall into 4 groups of 16,
// each group covering one row's 32 keys (kt) or 32 dims (v).  With 16-byte
// aligned pitches the group starts land 0, 32, 0, 32 banks apart; GP extra
// halves after every 16 rows move them to 0, 32, 16, 48 and keep every row
// 16-byte aligned for the operand reads.  Kept at d_k 128 only, where it
// measured faster (d_k 64: slightly slower).
template <int D>
struct DqSmem {
  static constexpr int RP = D + 8;   // fp16 pitch of [key][d] rows
  static constexpr int TP = MB + 8;  // fp16 pitch of [d][key] rows
  static constexpr int GP = D == 128 ? 32 : 0;  // halves after every 16 rows of kt and v
  f16 k[2][MB * RP];                 // [buffer]
  f16 kt[2][D * TP + GP * (D / 16)];
  f16 v[2][MB * RP + GP * (MB / 16)];
};

// dq and the per-query statistics (lse2, D) for the key-stationary kernel.
// Workgroup: 128 queries of one (batch, head), a wave per 32; key blocks of 32
// staged per source into a double LDS buffer (the next pass is staged while
// the current one is computed, one barrier per pass).  S^T = K Q^T keeps a
// query per lane; dP^T = V dO^T; dS^T = P^T (dP^T - D); dQ^T += K^T dS^T.
template <int D, bool BUF>
__global__ __launch_bounds__(256, D == 64 ? 3 : 2) void bwd_dq_mfma(BwdProblem p) {
  constexpr int NS = D / 16, NB = D / 32;
  constexpr int RP = DqSmem<D>::RP, TP = DqSmem<D>::TP, GP = DqSmem<D>::GP;
  __shared__ DqSmem<D> sm;
  const int N = p.N, H = p.H, w = p.w, BH = p.B * p.H;
  const int nQT = (N + MQ - 1) / MQ;
  const int qt = nQT - 1 - (int)(blockIdx.x / BH);  // longest first
  const int bh = (int)(blockIdx.x % BH), b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, lr = lane & 31, lg = lane >> 5;
  const int q0 = qt * MQ, qw0 = q0 + 32 * wave, qi = qw0 + lr;
  const int qc = qi < N ? qi : N - 1;
  const f16* Qp = (const f16*)p.Q + (size_t)bh * N * D;
  const f16* const Kl = (const f16*)p.K_loc + (size_t)bh * N * D;
  const f16* const Kg = (const f16*)p.K_glob + (size_t)bh * N * D;
  const f16* const Vl = (const f16*)p.V_loc + (size_t)bh * D * N;
  const f16* const Vg = (const f16*)p.V_glob + (size_t)bh * D * N;
  auto Kp = [&](int src) { return src ? Kg : Kl; };  // source 0 local, 1 global
  auto Vp = [&](int src) { return src ? Vg : Vl; };
  const float sc2 = kLog2e / sqrtf((float)D);

  f16x8 qf[NS], gf[NS];
  float Dd = 0.f;
  {
    const size_t orow = ((size_t)b * N + qc) * (size_t)(H * D) + (size_t)h * D;
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int d0 = 16 * st + 8 * lg;
      qf[st] = *(const f16x8*)(Qp + (size_t)qc * D + d0);
      const u32x4 g = *(const u32x4*)((const bf16*)p.dO + orow + d0);
      const u32x4 o = *(const u32x4*)((const bf16*)p.o + orow + d0);
      gf[st] = __builtin_bit_cast(f16x8, bf16x8_to_f16x8(g));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Dd = fmaf(__uint_as_float(g[e] << 16), __uint_as_float(o[e] << 16), Dd);
        Dd = fmaf(__uint_as_float(g[e] & 0xffff0000u), __uint_as_float(o[e] & 0xffff0000u), Dd);
      }
    }
  }
  Dd += __shfl_xor(Dd, 32);  // the other half of the dims

  const int i_last = min(q0 + MQ, N) - 1;
  auto need = [&](int src, int j0) {  // does any wave of the workgroup have pairs here?
    const int dmax = i_last - j0, dmin = q0 - min(j0 + 31, N - 1);
    if (dmax < 0) return false;
    return src == 0 ? (w > 0 && max(dmin, 0) < w) : dmax >= w;
  };
  // Passes: for each key block, the global source (if needed) then the local
  // one; every block j0 <= i_last needs at least one.
  auto next_pass = [&](int& j0, int& src) {
    if (src == 1 && need(0, j0)) {
      src = 0;
    } else {
      j0 += MB;
      src = need(1, j0) ? 1 : 0;
    }
  };
  auto scores = [&](f32x16& s, int bf) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int st = 0; st < NS; ++st)
      s = mfma32x32x16(*(const f16x8*)(sm.k[bf] + row_perm(lr) * RP + 16 * st + 8 * lg), qf[st],
                       s);
  };
  auto mask = [&](f32x16& s, int src, int j0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = j0 + perm_row(r, lg);
      s[r] = ((j < N) & keep_pair(src, qi - j, w)) ? s[r] : -INFINITY;
    }
  };

  // lse2 of each query: the forward's, or sweep 1 (maximum and sum per lane
  // half, then combined)
  float lse2;
  if (p.lse_in != nullptr) {
    lse2 = p.lse_in[(size_t)bh * N + qc] * kLog2e;
  } else {
    float m = -INFINITY, l = 0.f;
    {
      int j0 = 0, src = need(1, 0) ? 1 : 0, bf = 0;
      Rows<D> kx;
      load_rows<D>(kx, Kp(src), j0, N);
      store_rows<D, RP>(kx, sm.k[bf]);
      __syncthreads();
      while (true) {
        int nj0 = j0, nsrc = src;
        next_pass(nj0, nsrc);
        const bool has_next = nj0 <= i_last;
        if (has_next) load_rows<D>(kx, Kp(nsrc), nj0, N);  // in flight during the pass
        const BlockPass bp = block_pass(src, qw0, j0, N, w);
        if (bp.part) {
          f32x16 s;
          scores(s, bf);
          if (bp.masked) mask(s, src, j0);
          float mt = -INFINITY;
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[r]);
          mt *= sc2;
          const float m_new = fmaxf(m, mt);
          if (m_new > -INFINITY) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -m_new));
            l = l * __builtin_amdgcn_exp2f(m - m_new) + acc;
            m = m_new;
          }
        }
        if (has_next) store_rows<D, RP>(kx, sm.k[bf ^ 1]);
        __syncthreads();
        if (!has_next) break;
        j0 = nj0;
        src = nsrc;
        bf ^= 1;
      }
    }
    {
      const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
      const float mm = fmaxf(m, mo);
      l = (m > -INFINITY ? l * __builtin_amdgcn_exp2f(m - mm) : 0.f) +
          (mo > -INFINITY ? lo * __builtin_amdgcn_exp2f(mo - mm) : 0.f);
      m = mm;
    }
    lse2 = m + __log2f(l);
  }
  if (qi < N && lg == 0) {
    p.lse[(size_t)bh * N + qi] = lse2;
    p.Dd[(size_t)bh * N + qi] = Dd;
  }

  // sweep 2: dQ^T += K^T (P^T (dP^T - D))
  f32x16 dq[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;
  {
    int j0 = 0, src = need(1, 0) ? 1 : 0, bf = 0;
    // threads 0 .. 127 stage K (rows and transposed), 128 .. 255 V (as rows)
    const bool kside = tid < 128;
    const int pi = tid & 127;
    Pairs<D, MB> px;
    auto load2 = [&](int jj, int ss) {
      if (kside) load_pairs<D, MB, BUF>(px, Kp(ss), 0, jj, N, pi);
      else load_vt_pairs<D>(px, Vp(ss), jj, N, pi);
    };
    auto store2 = [&](int bb) {
      if (kside) store_pairs<D, MB, RP, TP, false, GP>(px, sm.k[bb], sm.kt[bb], pi);
      else store_vt_pairs<D, RP, GP>(px, sm.v[bb], pi);
    };
    load2(j0, src);
    store2(bf);
    __syncthreads();
    while (true) {
      int nj0 = j0, nsrc = src;
      next_pass(nj0, nsrc);
      const bool has_next = nj0 <= i_last;
      if (has_next) load2(nj0, nsrc);  // in flight during the pass
      const BlockPass bp = block_pass(src, qw0, j0, N, w);
      if (bp.part) {
        f32x16 s, dp;
        scores(s, bf);
        if (bp.masked) mask(s, src, j0);
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
        for (int st = 0; st < NS; ++st)
          dp = mfma32x32x16(*(const f16x8*)(sm.v[bf] + row_perm(lr) * RP +
                                            GP * (row_perm(lr) >> 4) + 16 * st + 8 * lg),
                            gf[st], dp);
        f16x8 dsb[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], sc2, -lse2));
          dsb[r >> 3][r & 7] = (f16)(pr * (dp[r] - Dd));
        }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int db = 0; db < NB; ++db)
            dq[db] = mfma32x32x16(
                *(const f16x8*)(sm.kt[bf] + (32 * db + lr) * TP + GP * (2 * db + (lr >> 4)) +
                                16 * u + 8 * lg),
                dsb[u],
                dq[db]);
      }
      if (has_next) store2(bf ^ 1);
      __syncthreads();
      if (!has_next) break;
      j0 = nj0;
      src = nsrc;
      bf ^= 1;
    }
  }
  if (qi < N) {
    const float sc = 1.f / sqrtf((float)D);
    float* out = p.dQ + ((size_t)bh * N + qi) * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = 32 * db + 8 * a + 4 * lg;
        *(float4*)(out + d) = make_float4(dq[db][4 * a] * sc, dq[db][4 * a + 1] * sc,
                                          dq[db][4 * a + 2] * sc, dq[db][4 * a + 3] * sc);
      }
  }
}

template <int D>
struct DkvSmem {
  static constexpr int QB = 64;      // queries per staged block (two 32-row sub-blocks)
  static constexpr int RP = D + 8;   // fp16 pitch of [query][d] rows
  static constexpr int TP = QB + 8;  // fp16 pitch of [d][query] rows
  f16 q[2][QB * RP];                 // [buffer]
  f16 qt[2][D * TP];
  f16 g[2][QB * RP];
  f16 gt[2][D * TP];
  float lse[2][QB], Dd[2][QB];
};

// dK and dV of each source.  Workgroup: 128 keys of one (batch, head), 32 per
// wave; query blocks of 64 (Q, dO, lse2, D) staged into a double LDS buffer
// and taken as two 32-query sub-blocks, one sweep per source.  S = Q K^T keeps
// a key per lane; P = 2^(S sc2 - lse2); dP = dO V^T; dS = P (dP - D);
// dV^T += dO^T P; dK^T += Q^T dS.
// The next block is staged in two halves of its head dims (all 64 queries
// each, so half a block of registers is in flight; a wave's transposed stores
// then cover 32 row pairs in two column groups 32 banks apart, without
// conflicts).  The dV/dK operands are read ahead of their MFMAs.
// ROLE 0: a wave computes both dV and dK of its 32 keys (4 waves).  ROLE 1 and
// 2 split them over two waves that share the staged blocks: ROLE 1 stages the
// blocks and forms S, P and dV; ROLE 2 forms S, dP, dS and dK.  S is then
// computed twice, but each wave holds one accumulator instead of two, which
// at d_k 128 is the difference between one and two waves per SIMD.
constexpr int kDkvBoth = 0, kDkvV = 1, kDkvK = 2;

template <int D, bool BUF, int ROLE>
__device__ __forceinline__ void dkv_role(const BwdProblem& p, DkvSmem<D>& sm, int wave) {
  constexpr int NS = D / 16, NB = D / 32;
  constexpr int RP = DkvSmem<D>::RP, TP = DkvSmem<D>::TP, QB = DkvSmem<D>::QB;
  constexpr bool DOV = ROLE != kDkvK, DOK = ROLE != kDkvV;  // this wave's accumulators
  constexpr bool STAGE = ROLE != kDkvK;                     // this wave stages blocks
  const int N = p.N, H = p.H, w = p.w, BH = p.B * p.H;
  const int kt = (int)(blockIdx.x / BH);  // small key tiles (most queries) first
  const int bh = (int)(blockIdx.x % BH), b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int k0 = kt * MQ, kw0 = k0 + 32 * wave, kj = kw0 + lr;
  const int kc = kj < N ? kj : N - 1;
  const f16* Qp = (const f16*)p.Q + (size_t)bh * N * D;
  const float sc2 = kLog2e / sqrtf((float)D), sc = 1.f / sqrtf((float)D);
  const int k_last = min(k0 + MQ, N) - 1;

  const bf16* Gp = (const bf16*)p.dO + (size_t)b * N * (size_t)(H * D) + (size_t)h * D;
  // threads 0 .. 127 stage Q, 128 .. 255 dO (rows and transposed)
  const bool qside = tid < 128;
  const int pi = tid & 127;
  constexpr int DC = D / 2;  // head dims per staged half of a block (all its queries)
  Pairs<DC, QB> px;
  float lx = 0.f, dx = 0.f;
  auto load = [&](int i0, int hf) {
    if constexpr (!STAGE) return;
    if (qside) load_pairs<DC, QB, BUF, D>(px, Qp + DC * hf, 0, i0, N, pi);
    else load_pairs<DC, QB, BUF>(px, Gp + DC * hf, (size_t)(H * D), i0, N, pi);
    if (hf == 0 && tid < QB) {  // staged as the initial values of the S and dP accumulators
      const int i = i0 + tid;
      lx = i < N ? -p.lse[(size_t)bh * N + i] / sc2 : 0.f;
      dx = i < N ? -p.Dd[(size_t)bh * N + i] : 0.f;
    }
  };
  auto store = [&](int bf, int hf) {
    if constexpr (!STAGE) return;
    if (qside) store_pairs<DC, QB, RP, TP>(px, sm.q[bf] + DC * hf, sm.qt[bf] + DC * hf * TP, pi);
    else store_pairs<DC, QB, RP, TP, true>(px, sm.g[bf] + DC * hf, sm.gt[bf] + DC * hf * TP, pi);
    if (hf == 0 && tid < QB) {
      sm.lse[bf][tid] = lx;
      sm.Dd[bf][tid] = dx;
    }
  };

#pragma unroll 1
  for (int src = 0; src < 2; ++src) {
    const f16* Kp = (const f16*)(src ? p.K_glob : p.K_loc) + (size_t)bh * N * D;
    const f16* Vp = (const f16*)(src ? p.V_glob : p.V_loc) + (size_t)bh * D * N;
    f16x8 kf[NS], vf[DOK ? NS : 1];  // this lane's key, dims 16 st + 8 lg .. +8
#pragma unroll
    for (int st = 0; st < NS; ++st)
      kf[st] = *(const f16x8*)(Kp + (size_t)kc * D + 16 * st + 8 * lg);
    if constexpr (DOK) {
      // V is [d][n] per (batch, head), the key a column of it: a per-lane base
      // and wave-uniform row offsets.  Indexed as (16 st + 8 lg + e) N + kc
      // instead, the compiler hoists one 64-bit offset per element out of the
      // source loop, NS * 8 register pairs held through the whole kernel.
      const f16* vcol = Vp + (size_t)(8 * lg) * N + kc;
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int e = 0; e < 8; ++e) vf[st][e] = vcol[(size_t)(16 * st + e) * N];
    }
    f32x16 dvt[DOV ? NB : 1], dkt[DOK ? NB : 1];
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DOV) dvt[db][r] = 0.f;
        if constexpr (DOK) dkt[db][r] = 0.f;
      }
    // queries with a pair of this source for some key of the workgroup
    const int i_begin = src == 0 ? k0 : min(N, k0 + w) / MB * MB;
    const int i_end = src == 0 ? min(N, k_last + w) : N;
    if (i_begin < i_end) {
      int i0 = i_begin, bf = 0;
      load(i0, 0);
      store(bf, 0);
      load(i0, 1);
      store(bf, 1);
      __syncthreads();
      while (true) {
        const bool has_next = i0 + QB < i_end;
        if (has_next) load(i0 + QB, 0);  // in flight during the first sub-block
#pragma unroll 1
        for (int sb = 0; sb < 2; ++sb) {
          const int q0 = i0 + 32 * sb;  // first query of the sub-block
          const BlockPass bp = block_pass(src, q0, kw0, N, w);
          if (sb == 1 && has_next) {  // the other buffer is not read in this block
            store(bf ^ 1, 0);
            load(i0 + QB, 1);
          }
          if (!bp.part) continue;
          // S - lse2/sc2 and dP - D: the accumulators start from the staged
          // per-query values, so P = 2^(S sc2) and dS = P dP afterwards
          f32x16 s, dp;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[r] = sm.lse[bf][32 * sb + perm_row(r, lg)];
            if constexpr (DOK) dp[r] = sm.Dd[bf][32 * sb + perm_row(r, lg)];
          }
          const int arow = (32 * sb + row_perm(lr)) * RP + 8 * lg;
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            s = mfma32x32x16(*(const f16x8*)(sm.q[bf] + arow + 16 * st), kf[st], s);
            if constexpr (DOK)
              dp = mfma32x32x16(*(const f16x8*)(sm.g[bf] + arow + 16 * st), vf[st], dp);
          }
          // the staged lse/D values and the first four operands are read
          // before the MFMAs start, then one more after each MFMA
          constexpr int NM = DOK ? 2 * NS : NS;  // MFMAs of the scores (and dP)
          __builtin_amdgcn_sched_group_barrier(0x100, (DOK ? 16 : 8) + 4, 0);
#pragma unroll
          for (int k = 0; k < NM - 4; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
          // dV/dK operands of the first 16 queries, read before the
          // exponentials so that their LDS latency hides under them
          const int tb = lr * TP + 32 * sb + 8 * lg;
          // (16-byte aligned: every term is a multiple of 8 halves; stated, or
          // the reads below are split into 4-byte accesses that conflict)
          const f16* gtb = (const f16*)__builtin_assume_aligned(sm.gt[bf] + tb, 16);
          const f16* qtb = (const f16*)__builtin_assume_aligned(sm.qt[bf] + tb, 16);
          f16x8 ga[DOV ? NB : 1], qa[DOK ? NB : 1];
#pragma unroll
          for (int db = 0; db < NB; ++db) {
            if constexpr (DOV) ga[db] = *(const f16x8*)(gtb + 32 * db * TP);
            if constexpr (DOK) qa[db] = *(const f16x8*)(qtb + 32 * db * TP);
          }
          f16x8 pb[2], dsb[2];
          if (bp.masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int i = q0 + perm_row(r, lg);
              float pr = __builtin_amdgcn_exp2f(s[r] * sc2);
              pr = ((i < N) & (kj < N) & keep_pair(src, i - kj, w)) ? pr : 0.f;
              if constexpr (DOV) pb[r >> 3][r & 7] = (f16)pr;
              if constexpr (DOK) dsb[r >> 3][r & 7] = (f16)(pr * dp[r]);
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pr = __builtin_amdgcn_exp2f(s[r] * sc2);
              if constexpr (DOV) pb[r >> 3][r & 7] = (f16)pr;
              if constexpr (DOK) dsb[r >> 3][r & 7] = (f16)(pr * dp[r]);
            }
          }
          {
            // the second 16 queries' operands, read while the first ones' MFMAs run
            f16x8 gb[DOV ? NB : 1], qb[DOK ? NB : 1];
#pragma unroll
            for (int db = 0; db < NB; ++db) {
              if constexpr (DOV) gb[db] = *(const f16x8*)(gtb + 32 * db * TP + 16);
              if constexpr (DOK) qb[db] = *(const f16x8*)(qtb + 32 * db * TP + 16);
            }
#pragma unroll
            for (int db = 0; db < NB; ++db) {
              if constexpr (DOV) dvt[db] = mfma32x32x16(ga[db], pb[0], dvt[db]);
              if constexpr (DOK) dkt[db] = mfma32x32x16(qa[db], dsb[0], dkt[db]);
            }
#pragma unroll
            for (int db = 0; db < NB; ++db) {
              if constexpr (DOV) dvt[db] = mfma32x32x16(gb[db], pb[1], dvt[db]);
              if constexpr (DOK) dkt[db] = mfma32x32x16(qb[db], dsb[1], dkt[db]);
            }
          }
        }
        if (has_next) store(bf ^ 1, 1);
        __syncthreads();
        if (!has_next) break;
        i0 += QB;
        bf ^= 1;
      }
    }
    if (kj < N) {
      float* dK = (src ? p.dK_glob : p.dK_loc) + ((size_t)bh * N + kj) * D;
      float* dV = (src ? p.dV_glob : p.dV_loc) + ((size_t)bh * N + kj) * D;
#pragma unroll
      for (int db = 0; db < NB; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int d = 32 * db + 8 * a + 4 * lg;
          if constexpr (DOK)
            *(float4*)(dK + d) = make_float4(dkt[db][4 * a] * sc, dkt[db][4 * a + 1] * sc,
                                             dkt[db][4 * a + 2] * sc, dkt[db][4 * a + 3] * sc);
          if constexpr (DOV)
            *(float4*)(dV + d) = make_float4(dvt[db][4 * a], dvt[db][4 * a + 1],
                                             dvt[db][4 * a + 2], dvt[db][4 * a + 3]);
        }
    }
  }
}

template <int D, bool BUF>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void bwd_dkv_mfma(BwdProblem p) {
  __shared__ DkvSmem<D> sm;
  dkv_role<D, BUF, kDkvBoth>(p, sm, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6));
}

// The same work on 8 waves: waves 0-3 stage and accumulate dV, waves 4-7
// accumulate dK of the same keys (two waves per SIMD, one of each role).
template <int D, bool BUF>
__global__ __launch_bounds__(512, 1) void bwd_dkv_split(BwdProblem p) {
  __shared__ DkvSmem<D> sm;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // block tests are scalar
  if (wave < 4)
    dkv_role<D, BUF, kDkvV>(p, sm, wave);
  else
    dkv_role<D, BUF, kDkvK>(p, sm, wave - 4);
}

}  // namespace

size_t attn_backward_workspace_bytes(int B, int N, int H) {
  const size_t one = ((sizeof(float) * (size_t)B * H * N) + 255) & ~(size_t)255;
  return 2 * one;
}

hipError_t launch_attn_backward(const BwdProblem& p_in, dar_dtype dt, hipStream_t s) {
  // Distances never exceed N - 1: any w >= N selects the local source for every pair.
  BwdProblem p = p_in;
  if (p.w > p.N) p.w = p.N;
  const int BH = p.B * p.H;
  const int nQT = (p.N + BQ - 1) / BQ;
  const int nKT = (p.N + 256 / (p.d_k / 16) - 1) / (256 / (p.d_k / 16));
  const dim3 g1(nQT * BH), g2(nKT * BH);
#define DAR_BWD(BFV, DV)                                                   \
  do {                                                                     \
    hipLaunchKernelGGL((bwd_dq<BFV, DV>), g1, dim3(256), 0, s, p);         \
    hipLaunchKernelGGL((bwd_dkv<BFV, DV>), g2, dim3(256), 0, s, p);        \
  } while (0)
  const bool bf = dt == DAR_BF16;
  if (bf) {
    const int nT = (p.N + MQ - 1) / MQ;
    // buffer-resource staging when the largest staged array (one batch's dO
    // rows, stride heads * d_k) is under 2 GiB
    const bool buf = (long)p.N * p.H * p.d_k * 2 < 0x7fffffffL;
    // d_k 64: one wave per 32 keys holds both accumulators at two waves per
    // SIMD; d_k 128: the split kernel (dV and dK on separate waves)
#define DAR_BWD_MFMA(DV, BUFV, KV, NT)                                                \
  do {                                                                            \
    hipLaunchKernelGGL((bwd_dq_mfma<DV, BUFV>), dim3(nT * BH), dim3(256), 0, s, p); \
    hipLaunchKernelGGL((KV<DV, BUFV>), dim3(nT * BH), dim3(NT), 0, s, p);           \
  } while (0)
    if (p.d_k == 64) {
      if (buf) DAR_BWD_MFMA(64, true, bwd_dkv_mfma, 256);
      else DAR_BWD_MFMA(64, false, bwd_dkv_mfma, 256);
    } else {
      if (buf) DAR_BWD_MFMA(128, true, bwd_dkv_split, 512);
      else DAR_BWD_MFMA(128, false, bwd_dkv_split, 512);
    }
#undef DAR_BWD_MFMA
  } else if (p.d_k == 64) {
    DAR_BWD(false, 64);
  } else {
    DAR_BWD(false, 128);
  }
#undef DAR_BWD
  return hipGetLastError();
}

}  // namespace dar
