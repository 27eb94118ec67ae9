// Projection GEMMs of the DAR layer.
//
// "Dual Dimensionality for Local and Global Attention":
//   Eq. (1)  h^D = h W_down
//   Eq. (3)  local  k = RoPE(h W_K),   v = h W_V;   q = h W_Q (text after Eq. 4)
//   Eq. (2)+(3) global k = RoPE(h' W_K), v = h' W_V with h' = h^D W_up, computed
//            as h^D (W_up W_K) and h^D (W_up W_V) once the weights are folded.
// All of these are GEMMs C = A B with A = activations [M, K] (row-major) and
// B a column-major weight, i.e. B^T stored row-major [width, K].  One launch
// covers several weights side by side ("segments"), each with its own output
// tensor and layout; the epilogue applies RoPE and scatters into the
// head-major layouts the attention kernels read.
//
// bf16 path: 128x128x64 tiles, 4 waves of 64x64 built from 32x32x16 MFMAs,
// double-buffered LDS, fp32 accumulate, epilogue staged through LDS so the
// rotate-half partners (t, t + d_k/2) meet in one thread and stores coalesce.
// fp32 path: an LDS-tiled VALU GEMM with the same epilogue (no bf16 anywhere).
#include "dar_common.hpp"

namespace dar {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA_S = BK + 8;  // bf16 per LDS row: 144 B, rows land 4 banks apart
constexpr int EPI_P = BN + 4;  // fp32 per epilogue row

struct SegTiles {
  int tile0[5];  // first column tile of each segment, tile0[nseg] = total
};

__device__ __forceinline__ int find_seg(const SegTiles& st, int nseg, int ct) {
  int s = 0;
  while (s + 1 < nseg && ct >= st.tile0[s + 1]) ++s;
  return s;
}

// Writes a [rows x BN] fp32 tile held in LDS (pitch EPI_P) to segment `seg`.
// Tile row r is GEMM row row0 + r; tile column c is segment column col0 + c.
template <typename OutT>
__device__ void epilogue_store(const float* tile, int rows, int row0, int col0,
                               const GemmSeg& seg, const GemmProblem& p) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int M = p.M, width = seg.width;
  OutT* out = (OutT*)seg.out;
  if (seg.kind == kRowMajor) {
    for (int it = tid; it < rows * (BN / 4); it += nthr) {
      const int r = it / (BN / 4), c = (it % (BN / 4)) * 4;
      const int grow = row0 + r, gcol = col0 + c;
      if (grow >= M || gcol >= width) continue;
      const float* src = tile + r * EPI_P + c;
      OutT* dst = out + (size_t)grow * width + gcol;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = from_f32<OutT>(src[e]);
    }
    return;
  }
  const int D = p.d_k, H = p.heads, Nq = p.n_seq;
  if (seg.kind == kHead) {
    if (seg.rope) {
      const int half = D / 2;
      // one item = 4 columns t..t+3 of the first half of a head and their partners
      const int per_row = BN / 8;
      for (int it = tid; it < rows * per_row; it += nthr) {
        const int r = it / per_row, q = it % per_row;
        const int hl = (q * 4) / half;          // head within the tile
        const int t = (q * 4) % half;           // first-half column within the head
        const int c = hl * D + t;               // tile column of x
        const int grow = row0 + r, gcol = col0 + c;
        if (grow >= M || gcol >= width) continue;
        const int b = grow / Nq, n = grow % Nq, head = gcol / D;
        const int pos = p.pos0 + n;
        const float* x = tile + r * EPI_P + c;
        const float* y = x + half;
        OutT* dst = out + (((size_t)b * H + head) * Nq + n) * D + t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 cs = rope_cs(p.rope, pos, t + e);
          dst[e] = from_f32<OutT>(x[e] * cs.x - y[e] * cs.y);
          dst[e + half] = from_f32<OutT>(x[e] * cs.y + y[e] * cs.x);
        }
      }
    } else {
      for (int it = tid; it < rows * (BN / 4); it += nthr) {
        const int r = it / (BN / 4), c = (it % (BN / 4)) * 4;
        const int grow = row0 + r, gcol = col0 + c;
        if (grow >= M || gcol >= width) continue;
        const int b = grow / Nq, n = grow % Nq, head = gcol / D, t = gcol % D;
        const float* src = tile + r * EPI_P + c;
        OutT* dst = out + (((size_t)b * H + head) * Nq + n) * D + t;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = from_f32<OutT>(src[e]);
      }
    }
    return;
  }
  // kHeadT: out[b, head, t, n]; consecutive threads take consecutive rows n so
  // every scalar store of a wave is contiguous.
  for (int it = tid; it < rows * (BN / 4); it += nthr) {
    const int r = it % rows, c = (it / rows) * 4;
    const int grow = row0 + r, gcol = col0 + c;
    if (grow >= M || gcol >= width) continue;
    const int b = grow / Nq, n = grow % Nq;
    const float* src = tile + r * EPI_P + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int head = (gcol + e) / D, t = (gcol + e) % D;
      out[(((size_t)b * H + head) * D + t) * Nq + n] = from_f32<OutT>(src[e]);
    }
  }
}

// --------------------------------------------------------------------------
// bf16 MFMA GEMM.
__global__ __launch_bounds__(256, 2) void project_gemm_bf16(GemmProblem p, SegTiles st, int nM,
                                                           int nC, int nCp) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * BM * LDA_S * 2];
  // XCD-aware order: XCD x owns a contiguous group of column tiles (its slice
  // of the weights stays in that XCD's L2) and walks the row tiles in order,
  // so the row tile of h is read once per XCD.
  const int bid = blockIdx.x;
  const int x = bid % kNumXcd, k = bid / kNumXcd, g = nCp / kNumXcd;
  const int mt = k / g, ct = x * g + (k % g);
  if (ct >= nC || mt >= nM) return;
  const int s = find_seg(st, p.nseg, ct);
  const GemmSeg seg = p.seg[s];
  const int col0 = (ct - st.tile0[s]) * BN;  // first segment column of the tile
  const int row0 = mt * BM;
  const int K = p.K, M = p.M;
  const bf16* A = (const bf16*)p.A;
  const bf16* Bt = (const bf16*)seg.Bt;

  // LDS: [buf][A tile | B tile], each BM x LDA_S bf16
  bf16* const lds = (bf16*)smem;
  auto sA = [&](int buf) { return lds + (2 * buf) * BM * LDA_S; };
  auto sB = [&](int buf) { return lds + (2 * buf + 1) * BM * LDA_S; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;

  // global -> register staging: 4 x 16 B of A and of B per thread
  u32x4 ra[4], rb[4];
  auto load_regs = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = (tid & 7) * 8;
      const int ar = row0 + r, bc = col0 + r, kk = k0 + kc;
      u32x4 z = {0u, 0u, 0u, 0u};
      ra[i] = (ar < M && kk < K) ? *(const u32x4*)(A + (size_t)ar * K + kk) : z;
      rb[i] = (bc < seg.width && kk < K) ? *(const u32x4*)(Bt + (size_t)bc * K + kk) : z;
    }
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i, kc = (tid & 7) * 8;
      *(u32x4*)(sA(buf) + r * LDA_S + kc) = ra[i];
      *(u32x4*)(sB(buf) + r * LDA_S + kc) = rb[i];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + BK - 1) / BK;
  load_regs(0);
  store_lds(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_regs((kt + 1) * BK);
    const bf16* a_s = sA(cur) + (wm * 64 + lr) * LDA_S + 8 * lg;
    const bf16* b_s = sB(cur) + (wn * 64 + lr) * LDA_S + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *(const bf16x8*)(a_s + 32 * i * LDA_S + 16 * ks);
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = *(const bf16x8*)(b_s + 32 * j * LDA_S + 16 * ks);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_lds(cur ^ 1);
    __syncthreads();
  }

  // accumulators -> LDS tile (row-major fp32), then the layout-specific store
  float* tile = (float*)smem;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
        const int col = wn * 64 + 32 * j + lr;
        tile[row * EPI_P + col] = acc[i][j][r];
      }
  __syncthreads();
  epilogue_store<bf16>(tile, BM, row0, col0, seg, p);
}

// --------------------------------------------------------------------------
// fp32 VALU GEMM (fp32 mode and the weight fold).  B(k, n) = Bp[k*sbk + n*sbn].
constexpr int SM = 64, SK = 16;

template <typename InT, typename OutT>
__global__ __launch_bounds__(256) void gemm_simt(GemmProblem p, SegTiles st, long sbk, long sbn) {
  __shared__ float sAs[SK][SM + 4];
  __shared__ float sBs[SK][BN + 4];
  __shared__ float tile[SM * EPI_P];
  const int ct = blockIdx.x, mt = blockIdx.y;
  const int s = find_seg(st, p.nseg, ct);
  const GemmSeg seg = p.seg[s];
  const int col0 = (ct - st.tile0[s]) * BN, row0 = mt * SM;
  const InT* A = (const InT*)p.A;
  const InT* Bp = (const InT*)seg.Bt;
  const int K = p.K, M = p.M;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += SK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i, r = e / SK, kk = e % SK;
      const int gr = row0 + r, gk = k0 + kk;
      sAs[kk][r] = (gr < M && gk < K) ? to_f32(A[(size_t)gr * K + gk]) : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = tid + 256 * i;
      int n, kk;
      if (sbk == 1) {
        n = e / SK;
        kk = e % SK;
      } else {
        n = e % BN;
        kk = e / BN;
      }
      const int gn = col0 + n, gk = k0 + kk;
      sBs[kk][n] = (gn < seg.width && gk < K) ? to_f32(Bp[(size_t)gk * sbk + (size_t)gn * sbn])
                                              : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < SK; ++kk) {
      float a[4], b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sAs[kk][4 * ty + i];
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = sBs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[(4 * ty + i) * EPI_P + tx + 16 * j] = acc[i][j];
  __syncthreads();
  epilogue_store<OutT>(tile, SM, row0, col0, seg, p);
}

SegTiles seg_tiles(const GemmProblem& p) {
  SegTiles st{};
  int t = 0;
  for (int s = 0; s < p.nseg; ++s) {
    st.tile0[s] = t;
    t += (p.seg[s].width + BN - 1) / BN;
  }
  for (int s = p.nseg; s < 5; ++s) st.tile0[s] = t;
  return st;
}

}  // namespace

hipError_t launch_project_gemm(const GemmProblem& p, dar_dtype dt, hipStream_t s) {
  const SegTiles st = seg_tiles(p);
  const int nC = st.tile0[p.nseg];
  if (dt == DAR_BF16) {
    const int nM = (p.M + BM - 1) / BM;
    const int nCp = (nC + kNumXcd - 1) / kNumXcd * kNumXcd;
    hipLaunchKernelGGL(project_gemm_bf16, dim3(nM * nCp), dim3(256), 0, s, p, st, nM, nC, nCp);
  } else {
    const int nM = (p.M + SM - 1) / SM;
    hipLaunchKernelGGL((gemm_simt<float, float>), dim3(nC, nM), dim3(256), 0, s, p, st, 1L,
                       (long)p.K);
  }
  return hipGetLastError();
}

// Fold: out^T = W_KV^T W_up^T, i.e. rows n of W_KV^T ([hd, d] row-major, the
// column-major W_K / W_V) times W_up^T ([d, d_down] row-major, the column-major
// W_up).  out is [hd, d_down] row-major = column-major [d_down x hd].
hipError_t launch_fold(const void* W_up, const void* W_KV, void* out, int d, int d_down, int hd,
                       dar_dtype dt, hipStream_t s) {
  GemmProblem p{};
  p.A = W_KV;
  p.M = hd;
  p.K = d;
  p.nseg = 1;
  p.seg[0] = GemmSeg{W_up, out, d_down, kRowMajor, 0};
  p.n_seq = hd;
  p.heads = 1;
  p.d_k = 2;
  const SegTiles st = seg_tiles(p);
  const int nC = st.tile0[1], nM = (hd + SM - 1) / SM;
  if (dt == DAR_BF16)
    hipLaunchKernelGGL((gemm_simt<bf16, bf16>), dim3(nC, nM), dim3(256), 0, s, p, st,
                       (long)d_down, 1L);
  else
    hipLaunchKernelGGL((gemm_simt<float, float>), dim3(nC, nM), dim3(256), 0, s, p, st,
                       (long)d_down, 1L);
  return hipGetLastError();
}

}  // namespace dar
