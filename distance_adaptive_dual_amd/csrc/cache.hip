// Decode cache from a prefill.
//
// "Dual Dimensionality for Local and Global Attention": after a prompt is
// prefilled, generation continues with each past token used through exactly
// one path (the remark after Eq. (5)): the latent h^D_j of every position
// (Eq. 1) and the full keys/values of the w most recent positions only.  The
// prefill hands its projections over in the attention kernel's formats (fp16;
// V transposed per head); the decode cache is bf16, latents [B, cap, d_down]
// and a ring [B, heads, w, d_k] indexed by position mod w.  Two kernels copy
// and convert: one for the latent rows, one for the ring (V through an LDS
// transpose).
#include "dar_common.hpp"

namespace dar {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ u32x4 f16x8_to_bf16x8(const u32x4& v) {
  const h8 x = __builtin_bit_cast(h8, v);
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_bf16x2((float)x[2 * e], (float)x[2 * e + 1]);
  return r;
}

// Packed prompts: the prompt b holding packed row r (the last b < nb with
// cu[b] <= r) and the row's position r - cu[b] in it.  The starts are read on
// the device only; for inconsistent values the result stays in [0, nb) and
// `ok` is false unless the row lies inside its prompt's [cu[b], cu[b+1]).
struct PackedRow { int b, n; bool ok; };
__device__ __forceinline__ PackedRow packed_row(const int* __restrict__ cu, int nb, int r) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int start = cu[lo], end = cu[lo + 1];
  return {lo, r - start, r >= start && r < end};
}

// h_D_cache[b, row0 + n, :] = bf16(h_D[b, n, :]) for n < N; 8 values per thread.
// Packed prompts (cu != null, B = 1, N = T rows): packed row r of prompt b at
// position n goes to h_D_cache[b, n, :] (n < cap), for b < nb.
__global__ __launch_bounds__(256) void latent_cast_kernel(const f16* __restrict__ hD,
                                                          bf16* __restrict__ cache, int B, int N,
                                                          int d_down, int cap, int row0,
                                                          const int* __restrict__ cu, int nb) {
  const int cpr = d_down / 8;  // 16-byte chunks per row
  const size_t total = (size_t)B * N * cpr;
  for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < total;
       c += (size_t)gridDim.x * blockDim.x) {
    const size_t row = c / cpr;
    const int col = (int)(c % cpr) * 8;
    size_t b = row / N, n = row % N;
    if (cu != nullptr) {
      const PackedRow L = packed_row(cu, nb, (int)row);
      if (!L.ok || L.n >= cap) continue;
      b = L.b;
      n = L.n;
    }
    const u32x4 v = *(const u32x4*)(hD + row * d_down + col);
    *(u32x4*)(cache + (b * cap + row0 + n) * d_down + col) = f16x8_to_bf16x8(v);
  }
}

// Ring slots of positions j0 .. j0+63 (clipped to [j_lo, N)) of one (b, head)
// from arrays holding positions base .. N-1 (len = N - base rows):
// K_win[b, h, j mod w, :] = bf16(K[b, h, j - base, :]) and
// V_win[b, h, j mod w, :] = bf16(Vt[b, h, :, j - base]).
// Ragged batches (lens != null, base 0): sequence b ends at lens[b] (clamped
// to [1, N]) and its last min(w, lens[b]) positions are written.
// Packed prompts (cu != null, base 0, N = T packed rows): prompt b's block of
// head-major rows starts at element cu[b] * heads * D ([heads, len_b, D] for K,
// [heads, D, len_b] for V), len_b = cu[b+1] - cu[b] (clamped into the T rows).
template <int D>
__global__ __launch_bounds__(256) void ring_fill_kernel(const f16* __restrict__ Kl,
                                                        const f16* __restrict__ Vl,
                                                        bf16* __restrict__ Kw,
                                                        bf16* __restrict__ Vw, int N, int w,
                                                        int j_lo, int base, int heads,
                                                        const int* __restrict__ lens,
                                                        const int* __restrict__ cu) {
  constexpr int TJ = 64, TP = TJ + 2;  // positions per tile; LDS pitch (f16)
  __shared__ f16 vt[D * TP];
  const int bh = blockIdx.x, tid = threadIdx.x;
  int len = N - base;
  int n_end = N, lo = j_lo;
  const f16* K;
  const f16* V;
  if (cu != nullptr) {
    const int b = bh / heads, hh = bh % heads;
    const int s = min(max(cu[b], 0), N);
    len = min(max(cu[b + 1], s), N) - s;
    n_end = len;
    lo = max(len - w, 0);
    K = Kl + ((size_t)s * heads + (size_t)hh * len) * D;
    V = Vl + ((size_t)s * heads + (size_t)hh * len) * D;
  } else {
    if (lens != nullptr) {
      const int l = lens[bh / heads];
      n_end = l < 1 ? 1 : (l > N ? N : l);
      lo = max(n_end - w, base);
    }
    K = Kl + (size_t)bh * len * D;
    V = Vl + (size_t)bh * D * len;
  }
  const int j0 = lo + TJ * blockIdx.y;
  const int nj = min(TJ, n_end - j0);
  if (nj <= 0) return;
  bf16* KW = Kw + (size_t)bh * w * D;
  bf16* VW = Vw + (size_t)bh * w * D;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  for (int c = tid; c < nj * CPR; c += 256) {
    const int r = c / CPR, col = (c % CPR) * 8;
    const int j = j0 + r;
    const u32x4 v = *(const u32x4*)(K + (size_t)(j - base) * D + col);
    *(u32x4*)(KW + (size_t)(j % w) * D + col) = f16x8_to_bf16x8(v);
  }
  // V^T tile: row t holds positions j0 .. j0+nj-1 (element reads: the rows of
  // V need not be 16-byte aligned at j0)
  for (int e = tid; e < D * TJ; e += 256) {
    const int t = e / TJ, r = e % TJ;
    vt[t * TP + r] = r < nj ? V[(size_t)t * len + (j0 - base) + r] : (f16)0.f;
  }
  __syncthreads();
  for (int c = tid; c < nj * CPR; c += 256) {
    const int r = c / CPR, t0 = (c % CPR) * 8;
    u32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      out[e] = pack_bf16x2((float)vt[(t0 + 2 * e) * TP + r], (float)vt[(t0 + 2 * e + 1) * TP + r]);
    *(u32x4*)(VW + (size_t)((j0 + r) % w) * D + t0) = out;
  }
}

// The other direction, for a prefill chunk: positions j0 .. j0+63 (clipped to
// [base, p0)) of the ring into the local arrays of positions base .. base+len-1
// (fp16; Vt token-innermost):  K[b, h, j - base, :] = K_win[b, h, j mod w, :],
// Vt[b, h, :, j - base] = V_win[b, h, j mod w, :] for the positions the ring
// holds (j > p0 - w), zeros below them (base may be rounded down to a tile).
template <int D>
__global__ __launch_bounds__(256) void ring_to_local_kernel(const bf16* __restrict__ Kw,
                                                            const bf16* __restrict__ Vw,
                                                            f16* __restrict__ Kl,
                                                            f16* __restrict__ Vl, int w, int base,
                                                            int p0, int len) {
  constexpr int TJ = 64;
  __shared__ f16 vt[TJ * (D + 2)];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int j0 = base + TJ * blockIdx.y;
  const int nj = min(TJ, p0 - j0);
  const bf16* KW = Kw + (size_t)bh * w * D;
  const bf16* VW = Vw + (size_t)bh * w * D;
  f16* K = Kl + (size_t)bh * len * D;
  f16* V = Vl + (size_t)bh * D * len;
  for (int e = tid; e < nj * D; e += 256) {
    const int r = e / D, t = e % D;
    const int j = j0 + r;
    // positions the ring no longer holds (j <= p0 - w) are written as zeros
    const bool held = j > p0 - w;
    K[(size_t)(j - base) * D + t] = held ? (f16)(float)KW[(size_t)(j % w) * D + t] : (f16)0.f;
    vt[r * (D + 2) + t] = held ? (f16)(float)VW[(size_t)(j % w) * D + t] : (f16)0.f;
  }
  __syncthreads();
  for (int e = tid; e < nj * D; e += 256) {
    const int t = e / nj, r = e % nj;
    V[(size_t)t * len + (j0 - base) + r] = vt[r * (D + 2) + t];
  }
}

}  // namespace

hipError_t launch_latent_cast(const void* h_D, int B, int N, int d_down, int cap, int row0,
                              void* h_D_cache, hipStream_t s, const int* cu, int nb) {
  const size_t chunks = (size_t)B * N * (d_down / 8);
  size_t blocks = (chunks + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(latent_cast_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const f16*)h_D, (bf16*)h_D_cache, B, N, d_down, cap, row0, cu, nb);
  return hipGetLastError();
}

hipError_t launch_ring_fill(const void* K, const void* Vt, int B, int heads, int d_k, int N,
                            int base, int w, void* K_win, void* V_win, hipStream_t s,
                            const int* lens) {
  const int j_lo = max(N - w, base);
  if (w <= 0 || j_lo >= N) return hipSuccess;
  // a ragged sequence writes at most min(w, N - base) positions as well
  const dim3 grid(B * heads, (N - j_lo + 63) / 64);
  if (d_k == 64)
    hipLaunchKernelGGL(ring_fill_kernel<64>, grid, dim3(256), 0, s, (const f16*)K,
                       (const f16*)Vt, (bf16*)K_win, (bf16*)V_win, N, w, j_lo, base, heads, lens,
                       nullptr);
  else
    hipLaunchKernelGGL(ring_fill_kernel<128>, grid, dim3(256), 0, s, (const f16*)K,
                       (const f16*)Vt, (bf16*)K_win, (bf16*)V_win, N, w, j_lo, base, heads, lens,
                       nullptr);
  return hipGetLastError();
}

hipError_t launch_ring_to_local(const void* K_win, const void* V_win, int B, int heads, int d_k,
                                int w, int base, int p0, int len, void* K, void* Vt,
                                hipStream_t s) {
  if (w <= 0 || base >= p0) return hipSuccess;
  const dim3 grid(B * heads, (p0 - base + 63) / 64);
  if (d_k == 64)
    hipLaunchKernelGGL(ring_to_local_kernel<64>, grid, dim3(256), 0, s, (const bf16*)K_win,
                       (const bf16*)V_win, (f16*)K, (f16*)Vt, w, base, p0, len);
  else
    hipLaunchKernelGGL(ring_to_local_kernel<128>, grid, dim3(256), 0, s, (const bf16*)K_win,
                       (const bf16*)V_win, (f16*)K, (f16*)Vt, w, base, p0, len);
  return hipGetLastError();
}

hipError_t launch_cache_from_prefill(const void* h_D, const void* K_loc, const void* V_loc,
                                     int B, int N, int heads, int d_k, int d_down, int w,
                                     int cap, void* h_D_cache, void* K_win, void* V_win,
                                     hipStream_t s, const int* lens) {
  hipError_t e = launch_latent_cast(h_D, B, N, d_down, cap, 0, h_D_cache, s);
  if (e == hipSuccess)
    e = launch_ring_fill(K_loc, V_loc, B, heads, d_k, N, 0, w, K_win, V_win, s, lens);
  return e;
}

hipError_t launch_cache_from_packed(const void* h_D, const void* K_loc, const void* V_loc,
                                    const int* cu, int B, int T, int max_len, int heads, int d_k,
                                    int d_down, int w, int cap, void* h_D_cache, void* K_win,
                                    void* V_win, hipStream_t s) {
  hipError_t e = launch_latent_cast(h_D, 1, T, d_down, cap, 0, h_D_cache, s, cu, B);
  if (e != hipSuccess || w <= 0) return e;
  // each prompt writes its last min(w, len_b) <= min(w, max_len) positions
  const dim3 grid(B * heads, (min(w, max_len) + 63) / 64);
  if (d_k == 64)
    hipLaunchKernelGGL(ring_fill_kernel<64>, grid, dim3(256), 0, s, (const f16*)K_loc,
                       (const f16*)V_loc, (bf16*)K_win, (bf16*)V_win, T, w, 0, 0, heads, nullptr,
                       cu);
  else
    hipLaunchKernelGGL(ring_fill_kernel<128>, grid, dim3(256), 0, s, (const f16*)K_loc,
                       (const f16*)V_loc, (bf16*)K_win, (bf16*)V_win, T, w, 0, 0, heads, nullptr,
                       cu);
  return hipGetLastError();
}

// Weight packing: the equations' W in R^{rows x cols}, stored row-major
// (element (k, n) at k * cols + n, the row-vector convention of Eqs. 1-4), into
// the library's column-major layout (element (k, n) at n * rows + k).  A plain
// transpose through a 64 x 64 LDS tile: reads run along n, writes along k, both
// coalesced.  The padded pitch (65 elements) spreads a column of the tile over
// the banks.
template <typename T>
__global__ __launch_bounds__(256) void pack_transpose_kernel(const T* __restrict__ src,
                                                             T* __restrict__ dst, int rows,
                                                             int cols) {
  __shared__ T tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = src[(size_t)r * cols + c];
  }
  __syncthreads();
#pragma unroll 4
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[tx][i];
  }
}

hipError_t launch_pack_weight(const void* W, int rows, int cols, int elem_bytes, void* out,
                              hipStream_t s) {
  const dim3 grid((cols + 63) / 64, (rows + 63) / 64);
  if (elem_bytes == 2)
    pack_transpose_kernel<unsigned short>
        <<<grid, 256, 0, s>>>((const unsigned short*)W, (unsigned short*)out, rows, cols);
  else
    pack_transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)W, (float*)out, rows, cols);
  return hipGetLastError();
}

}  // namespace dar
