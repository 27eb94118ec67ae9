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
// Two VALU kernels, fp32 arithmetic (the inputs are fp16 / bf16 in bf16 mode,
// fp32 in fp32 mode; the gradients are fp32):
//   bwd_dq:  64 queries per workgroup, four lanes per query (lane part pt owns
//            dims pt, pt + 4, ...).  Keys of both sources are staged 32 at a
//            time.  A first sweep forms lse_i (online maximum and sum), then
//            D_i and lse_i are stored for the second kernel and a second sweep
//            accumulates dq_i.
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

  // sweep 1: lse_i over j <= i
  float m = -INFINITY, l = 0.f;
  for (int j0 = 0; j0 <= i_last; j0 += BK) {
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
  if (p.d_k == 64) {
    if (bf) DAR_BWD(true, 64); else DAR_BWD(false, 64);
  } else {
    if (bf) DAR_BWD(true, 128); else DAR_BWD(false, 128);
  }
#undef DAR_BWD
  return hipGetLastError();
}

}  // namespace dar
