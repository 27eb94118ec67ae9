// Fused dual-source causal attention (prefill).
//
// "Dual Dimensionality for Local and Global Attention", Eq. (3)-(4): query i
// attends to every key j <= i; the pair uses the full-state key/value
// (K_loc, V_loc) when i - j < w and the bottleneck key/value (K_glob, V_glob)
// otherwise; o_i = softmax(q_i K_i^T / sqrt(d_k)) V_i.
//
// bf16 kernel (gfx950): one workgroup = 128 queries of one (batch, head), four
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
// fp32 kernel: VALU only, four lanes per query, per-key online softmax; it
// exists for the fp32 mode (1e-4 parity), never rounds to bf16.
#include <math.h>

#include "dar_common.hpp"

namespace dar {

namespace {

constexpr int QT = 128;  // queries per workgroup
constexpr int KT = 64;   // keys per tile

__device__ __forceinline__ int key_perm(int r) {  // swap bits 2 and 3
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D>
struct PrefillSmem {
  static constexpr int KP = D + 8;   // bf16 per K row (16 B pad: 4-bank shift per row)
  static constexpr int VP = KT + 8;  // bf16 per V^T row
  bf16 k[2][KT * KP];                // [source][key][d]
  bf16 v[2][D * VP];                 // [source][d][key]
};

// Stage one source's K tile [KT x D] and V^T tile [D x KT] into LDS.
template <int D>
__device__ __forceinline__ void stage_tile(bf16* sk, bf16* sv, const bf16* K, const bf16* Vt,
                                           int N, int j0, bool vec_ok) {
  constexpr int KP = PrefillSmem<D>::KP, VP = PrefillSmem<D>::VP;
  const int tid = threadIdx.x;
  constexpr int KCH = KT * D / 8;  // 16-byte chunks of the K tile
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int c = tid; c < KCH; c += 256) {
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const int j = j0 + row;
    const u32x4 val = (j < N) ? *(const u32x4*)(K + (size_t)j * D + col) : z;
    *(u32x4*)(sk + row * KP + col) = val;
  }
  constexpr int VCH = D * KT / 8;
  if (vec_ok) {
#pragma unroll
    for (int c = tid; c < VCH; c += 256) {
      const int d = c / (KT / 8), kc = (c % (KT / 8)) * 8;
      *(u32x4*)(sv + d * VP + kc) = *(const u32x4*)(Vt + (size_t)d * N + j0 + kc);
    }
  } else {  // ragged tail or N not a multiple of 8: element-wise with bounds
    const uint16_t* src = (const uint16_t*)Vt;
    uint16_t* dst = (uint16_t*)sv;
    for (int e = tid; e < D * KT; e += 256) {
      const int d = e / KT, kk = e % KT, j = j0 + kk;
      dst[d * VP + kk] = (j < N) ? src[(size_t)d * N + j] : (uint16_t)0;
    }
  }
}

// S^T for one 64-key tile: s[kb][r] is key j0 + 32kb + 16(r/8) + 8lg + (r%8).
template <int D>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[2], const bf16* sk, const bf16x8 (&qf)[D / 16],
                                            int lr, int lg) {
  constexpr int KP = PrefillSmem<D>::KP;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const bf16* base = sk + (32 * kb + key_perm(lr)) * KP + 8 * lg;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      acc = mfma32x32x16(*(const bf16x8*)(base + 16 * st), qf[st], acc);
    s[kb] = acc;
  }
}

// O^T += V^T P^T over one 64-key tile.  pf[u] holds keys j0 + 16u + 8lg + c.
template <int D>
__device__ __forceinline__ void tile_pv(f32x16 (&o)[D / 32], const bf16* sv, const bf16x8 (&pf)[4],
                                        int lr, int lg) {
  constexpr int VP = PrefillSmem<D>::VP;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const bf16* base = sv + (32 * db + lr) * VP + 8 * lg;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[db] = mfma32x32x16(*(const bf16x8*)(base + 16 * u), pf[u], o[db]);
  }
}

template <int D>
__global__ __launch_bounds__(256, 1) void attn_prefill_bf16(PrefillProblem p, int nQT, int remap) {
  __shared__ PrefillSmem<D> sm;
  const int N = p.N, H = p.H, BH = p.B * p.H, w = p.w;
  // Longest query tiles first; with remap, all tiles of one (batch, head) stay
  // on one XCD so its K/V prefix is shared through that XCD's L2.
  int qt, bh;
  {
    const int bid = blockIdx.x;
    if (remap) {
      const int x = bid % kNumXcd, k = bid / kNumXcd, per = BH / kNumXcd;
      const int bl = k / nQT;
      qt = nQT - 1 - (k % nQT);
      bh = bl * kNumXcd + x;
      (void)per;
    } else {
      qt = nQT - 1 - bid / BH;
      bh = bid % BH;
    }
  }
  const int b = bh / H, h = bh % H;
  const size_t kv_off = (size_t)bh * N * D;
  const bf16* Qp = (const bf16*)p.Q + kv_off;
  const bf16* Kl = (const bf16*)p.K_loc + kv_off;
  const bf16* Kg = (const bf16*)p.K_glob + kv_off;
  const bf16* Vl = (const bf16*)p.V_loc + kv_off;
  const bf16* Vg = (const bf16*)p.V_glob + kv_off;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  const int i0 = qt * QT, qw0 = i0 + 32 * wave;
  const int qi = qw0 + lr;  // this lane's query
  const int i_last = min(i0 + QT - 1, N - 1);
  const int wi_last = min(qw0 + 31, N - 1);

  bf16x8 qf[D / 16];
  {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      u32x4 v = (qi < N) ? *(const u32x4*)(Qp + (size_t)qi * D + 16 * st + 8 * lg) : z;
      qf[st] = __builtin_bit_cast(bf16x8, v);
    }
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = kLog2e / sqrtf((float)D);
  const bool nvec = (N % 8) == 0;

  const int j_end = min(N, i0 + QT);
  for (int j0 = 0; j0 < j_end; j0 += KT) {
    const int dmin = i0 - (j0 + KT - 1), dmax = i_last - j0;
    const bool need_loc = (w > 0) && (max(dmin, 0) < w);
    const bool need_glob = dmax >= w;
    const bool vec_ok = nvec && (j0 + KT <= N);
    __syncthreads();
    if (need_loc) stage_tile<D>(sm.k[0], sm.v[0], Kl, Vl, N, j0, vec_ok);
    if (need_glob) stage_tile<D>(sm.k[1], sm.v[1], Kg, Vg, N, j0, vec_ok);
    __syncthreads();

    const int wdmax = wi_last - j0, wdmin = qw0 - (j0 + KT - 1);
    if (qw0 >= N || wdmax < 0) continue;
    const bool wl = (w > 0) && (max(wdmin, 0) < w);
    const bool wgl = wdmax >= w;
    const bool masked = (wdmin < 0) || (j0 + KT > N);

    f32x16 s[2];
    if (wl && wgl) {
      f32x16 sg[2];
      tile_scores<D>(s, sm.k[0], qf, lr, lg);
      tile_scores<D>(sg, sm.k[1], qf, lr, lg);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = j0 + 32 * kb + 16 * (r >> 3) + 8 * lg + (r & 7);
          if (qi - j >= w) s[kb][r] = sg[kb][r];
        }
    } else {
      tile_scores<D>(s, wl ? sm.k[0] : sm.k[1], qf, lr, lg);
    }

    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * sc;
        if (masked) {
          const int j = j0 + 32 * kb + 16 * (r >> 3) + 8 * lg + (r & 7);
          if (j > qi || j >= N) v = -INFINITY;
        }
        s[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = exp2f(s[kb][r] - m_new);
        s[kb][r] = e;
        ls += e;
      }
    l_run = l_run * alpha + ls;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    if (wl && wgl) {
      bf16x8 pl[4], pg[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int j = j0 + 16 * u + 8 * lg + c;
          const float e = s[u >> 1][8 * (u & 1) + c];
          const bool loc = (qi - j) < w;
          pl[u][c] = (bf16)(loc ? e : 0.f);
          pg[u][c] = (bf16)(loc ? 0.f : e);
        }
      tile_pv<D>(o, sm.v[0], pl, lr, lg);
      tile_pv<D>(o, sm.v[1], pg, lr, lg);
    } else {
      bf16x8 pf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 8; ++c) pf[u][c] = (bf16)s[u >> 1][8 * (u & 1) + c];
      tile_pv<D>(o, wl ? sm.v[0] : sm.v[1], pf, lr, lg);
    }
  }

  if (qi >= N) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  bf16* out = (bf16*)p.o + ((size_t)b * N + qi) * (size_t)(H * D) + (size_t)h * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = 32 * db + 8 * rq + 4 * lg;
      u32x2 v;
      v[0] = pack_bf16x2(o[db][4 * rq + 0] * inv, o[db][4 * rq + 1] * inv);
      v[1] = pack_bf16x2(o[db][4 * rq + 2] * inv, o[db][4 * rq + 3] * inv);
      *(u32x2*)(out + d) = v;
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
  float* out = (float*)p.o + ((size_t)b * N + qi) * (size_t)(H * D) + (size_t)h * D;
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < E; ++e) out[pt + 4 * e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_attn_prefill(const PrefillProblem& p, dar_dtype dt, hipStream_t s) {
  const int BH = p.B * p.H;
  if (dt == DAR_BF16) {
    const int nQT = (p.N + QT - 1) / QT;
    const int remap = (BH % kNumXcd) == 0 ? 1 : 0;
    const dim3 grid(nQT * BH);
    if (p.d_k == 64)
      hipLaunchKernelGGL(attn_prefill_bf16<64>, grid, dim3(256), 0, s, p, nQT, remap);
    else
      hipLaunchKernelGGL(attn_prefill_bf16<128>, grid, dim3(256), 0, s, p, nQT, remap);
  } else {
    const dim3 grid((p.N + FQ - 1) / FQ, p.H, p.B);
    if (p.d_k == 64)
      hipLaunchKernelGGL(attn_prefill_f32<64>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_prefill_f32<128>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace dar
