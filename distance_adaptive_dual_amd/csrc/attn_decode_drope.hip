// Decode of the decoupled-RoPE variant: one query per sequence, streaming the
// latent cache.
//
// "Dual Dimensionality for Local and Global Attention" names MLA's decoupled
// rotary embedding as the way to an efficient implementation (the paragraph
// after the inference remark).  The variant, read as MLA's construction on
// Eqs. (1)-(4): every head's query and key carry a content part (Eq. (3)
// without rotation) and a rotary part of width d_R; the rotary key
// kR_j = RoPE_j(h_j W_KR) is one per token, shared by the heads and by both
// paths; s_ij = (qC_i . kC_j + qR_i . kR_j) / sqrt(d_k + d_R).
//
// No rotation sits between W_upK and the query any more, so the content score
// of a distant token is qC_a . (h^D_j W_upK_a) = (W_upK_a^T qC_a) . h^D_j:
// the fold is absorbed into the query once per step, and the cache stream
// reads [h^D_j ; kR_j] (d_down + d_R values per token) once for all heads.
//   absorb  -- qa[b, a] = scale [W_upK_a^T qC_a ; qR_a] in fp32, stored as two
//              bf16 parts (hi + lo), so the score MFMAs lose nothing to the
//              rounding of the query;
//   stream  -- per (batch, group of 16 heads, chunk of positions), two waves
//              each streaming half the chunk through their own LDS double
//              buffer (buffer loads with an LDS destination):
//              S^T = X Qa^T on 16x16x32 MFMAs (X rows = tokens), an online
//              softmax per head, acc[head, d_down] += P X_lat on 16x16x32
//              MFMAs.  The P operand is the score registers as they are; the
//              X_lat operand (eight tokens of one latent column per lane) is
//              read from the row-major block with ds_read_b64_tr_b16;
//   window  -- per (batch, head): the positions p-w+1 .. p, content keys and
//              values from the ring, rotary keys from the cache (in the same
//              launch as the absorb, which it does not need);
//   combine -- the latent decode's log-sum-exp merge and single lift by
//              W_upV (decode_combine).
// Scores are base-2 logits: log2(e) / sqrt(d_k + d_R) is folded into qa.
#include <math.h>

#include <algorithm>

#include "dar_common.hpp"

namespace dar {

namespace {

#ifndef DAR_STREAM_NB
#define DAR_STREAM_NB 2
#endif
#ifndef DAR_STREAM_TARGET
#define DAR_STREAM_TARGET 512
#endif
constexpr int kStreamNB = DAR_STREAM_NB;  // buffers per wave (d_down <= 256)
constexpr int DT = 32;              // tokens per streamed block
constexpr int DWAVES = 2;           // waves per stream workgroup (chunk split)
constexpr int DTARGET_WG = DAR_STREAM_TARGET;  // stream workgroups to aim for
constexpr float kTauD = 8.f;        // move the reference max only past 2^8 growth
constexpr float kNegBigD = -1e30f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Geometry of one decode step.
struct DropeGeom {
  int n_glob;     // latent positions 0 .. n_glob-1
  int n_hg;       // groups of 16 heads
  int n_chunks;   // chunks per (batch, head group)
  int chunk_len;  // positions per chunk (a multiple of DWAVES * DT)
  int qw;         // d_down + d_R: width of an absorbed query row
  int n_win;      // window pieces per (batch, head), each <= win_len positions
  int win_len;
};

DropeGeom drope_geom(const DropeDecodeProblem& p) {
  DropeGeom g{};
  const long pp = (long)p.ctx - 1;
  g.n_glob = (int)(pp - p.w + 1 > 0 ? pp - p.w + 1 : 0);
  g.n_hg = (p.H + 15) / 16;
  g.qw = p.d_down + p.d_R;
  int want = DTARGET_WG / (p.B * g.n_hg);
  if (want < 1) want = 1;
  const int unit = DWAVES * DT;
  int len = (g.n_glob + want - 1) / want;
  len = (len + unit - 1) / unit * unit;
  if (len < unit) len = unit;
  g.chunk_len = len;
  g.n_chunks = g.n_glob > 0 ? (g.n_glob + len - 1) / len : 1;
  const long nw = p.w > 0 ? pp - (pp - p.w + 1 > 0 ? pp - p.w + 1 : 0) + 1 : 0;
  g.n_win = nw > 0 ? (int)std::min<long>(64, (nw + 127) / 128) : 1;
  g.win_len = nw > 0 ? (int)((nw + g.n_win - 1) / g.n_win) : 1;
  return g;
}

// qa = scale [W_upK_a^T qC_a ; qR_a] split into bf16 hi + lo.  Blocks
// (h, by, bz) over (H, ceil(qw / 64), ceil(B / 4)), four waves: column
// t = 64 by + lane of the absorbed rows of four batches, the contraction over
// the head's d_k split between the waves (each a quarter, its loads all in
// flight) and summed through LDS.
template <int D, int DR>
__device__ __forceinline__ void absorb_block(const DropeDecodeProblem& p, const DropeGeom& g,
                                             bf16* qa_hi, bf16* qa_lo, int h, int by, int bz) {
  constexpr int NBT = 4, CQ = D / 4;
  __shared__ float qcs[NBT][D];
  __shared__ float red[4][NBT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = by * 64 + lane;
  const int DD = p.d_down;
  const float scl = kLog2e / sqrtf((float)(D + DR));
  const bf16* Wk = (const bf16*)p.W_upK + (size_t)h * D * DD;
  {
    const int b0 = bz * NBT;
    const int nb = min(NBT, p.B - b0);
    for (int e = threadIdx.x; e < NBT * D; e += 256) {
      const int bi = e / D, c = e % D;
      qcs[bi][c] = bi < nb ? (float)((const bf16*)p.qC)[((size_t)(b0 + bi) * p.H + h) * D + c]
                           : 0.f;
    }
    __syncthreads();
    float acc[NBT];
#pragma unroll
    for (int bi = 0; bi < NBT; ++bi) acc[bi] = 0.f;
    if (t < DD) {
      float wv[CQ];
#pragma unroll
      for (int i = 0; i < CQ; ++i) wv[i] = (float)Wk[(size_t)(wave * CQ + i) * DD + t];
#pragma unroll
      for (int i = 0; i < CQ; ++i)
#pragma unroll
        for (int bi = 0; bi < NBT; ++bi) acc[bi] = fmaf(wv[i], qcs[bi][wave * CQ + i], acc[bi]);
    }
#pragma unroll
    for (int bi = 0; bi < NBT; ++bi) red[wave][bi][lane] = acc[bi];
    __syncthreads();
    for (int bi = wave; bi < nb; bi += 4) {
      if (t < g.qw) {
        const size_t row = (size_t)(b0 + bi) * p.H + h;
        float a = t < DD ? red[0][bi][lane] + red[1][bi][lane] + red[2][bi][lane] + red[3][bi][lane]
                         : (float)((const bf16*)p.qR)[row * DR + (t - DD)];
        a *= scl;
        const bf16 hi = (bf16)a;
        qa_hi[row * g.qw + t] = hi;
        qa_lo[row * g.qw + t] = (bf16)(a - (float)hi);
      }
    }
    __syncthreads();  // qcs and red are rewritten for the next batches
  }
}

template <int DD, int DR, int NB>
struct StreamSmem {
  // [wave][buffer] blocks of DT tokens, rows of DD (latent) / DR (rotary)
  // bf16 stored with 16-byte chunk c of row r at slot c ^ (r mod slots)
  bf16 lat[DWAVES][NB][DT * DD];
  bf16 rot[DWAVES][NB][DT * DR];
};

template <int N>
__device__ __forceinline__ void wait_vm() {  // s_waitcnt vmcnt(N), other counters free
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

template <int D, int DD, int DR, int NB>
__global__ __launch_bounds__(DWAVES * 64) void drope_stream(DropeDecodeProblem p, DropeGeom g,
                                                            const bf16* qa_hi, const bf16* qa_lo,
                                                            float* part) {
  static_assert(NB == 2 || NB == 3, "two or three buffers per wave");
  __shared__ StreamSmem<DD, DR, NB> sm;
  constexpr int KL = DD / 32, KR = DR / 32;       // 32-wide contraction steps
  constexpr int SL = 2 * DD / 16, SR = 2 * DR / 16;  // 16-byte slots per row
  constexpr int NL = DT * DD * 2 / 1024;          // 1 KB load instructions per block
  constexpr int NR = DT * DR * 2 / 1024;
  static_assert(SL >= 16 && (SL & (SL - 1)) == 0, "latent rows of 16+ slots");
  static_assert(NR >= 1 && SR >= 4, "rotary block of at least one instruction");
  constexpr int NCT = DD / 16;                    // 16-column tiles of the accumulator

  const int wg = blockIdx.x;
  const int chunk = wg % g.n_chunks, bhg = wg / g.n_chunks;
  const int b = bhg / g.n_hg, hg = bhg % g.n_hg;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, gq = lane >> 4;
  const int sub = g.chunk_len / DWAVES;
  const int c0 = chunk * g.chunk_len;
  const int w0 = min(g.n_glob, c0 + wave * sub), w1 = min(g.n_glob, c0 + (wave + 1) * sub);
  const int nblk = (w1 - w0 + DT - 1) / DT;

  // absorbed query of head hg*16 + n as the B operand (contraction k-group gq)
  bf16x8 qh[KL + KR], ql[KL + KR];
  {
    const int head = hg * 16 + n;
    if (head < p.H) {
      const size_t off = ((size_t)b * p.H + head) * g.qw + 8 * gq;
#pragma unroll
      for (int ks = 0; ks < KL + KR; ++ks) {
        qh[ks] = *(const bf16x8*)(qa_hi + off + 32 * ks);
        ql[ks] = *(const bf16x8*)(qa_lo + off + 32 * ks);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KL + KR; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) qh[ks][e] = ql[ks][e] = (bf16)0.f;
    }
  }

  // Rows w0 .. w1-1 of this sequence; the resources' range returns zeros past w1.
  const size_t row0 = (size_t)b * p.cap + (w0 < w1 ? w0 : 0);
  const int nrows = w1 - w0;
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.h_D + row0 * DD), (short)0, nrows * DD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.KR + row0 * DR), (short)0, nrows * DR * 2, 0x00020000);
  auto issue = [&](int blk, int buf) {
    bf16* dl = sm.lat[wave][buf];
    bf16* dr = sm.rot[wave][buf];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int byte = i * 1024 + 16 * lane;  // where this lane's 16 bytes land
      const int r = byte / (2 * DD), s = (byte % (2 * DD)) / 16;
      const int c = s ^ (r & 15);             // the row's chunk kept at slot s
      const unsigned off = (unsigned)(((blk * DT + r) * DD) * 2 + 16 * c);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rl, (__attribute__((address_space(3))) void*)(dl + i * 512), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int byte = i * 1024 + 16 * lane;
      const int r = byte / (2 * DR), s = (byte % (2 * DR)) / 16;
      const int c = s ^ (r & (SR - 1));
      const unsigned off = (unsigned)(((blk * DT + r) * DR) * 2 + 16 * c);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rr, (__attribute__((address_space(3))) void*)(dr + i * 512), 16, off, 0, 0, 0);
    }
  };

  float m_ref = kNegBigD, l_lane = 0.f;  // head n: reference max, this lane's share of the sum
  f32x4 acc[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int blk, int buf) {
    const bf16* L = sm.lat[wave][buf];
    const bf16* R = sm.rot[wave][buf];
    // scores: tile t holds tokens 16 t + 4 gq + i (register i) of head n
    f32x4 sh[2], sl[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) sh[t] = sl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KL; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = 16 * t + n, c = 4 * ks + gq;
        const bf16x8 a = *(const bf16x8*)(L + row * DD + 8 * (c ^ (row & 15)));
        sh[t] = mfma16(a, qh[ks], sh[t]);
        sl[t] = mfma16(a, ql[ks], sl[t]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < KR; ++ks) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = 16 * t + n, c = 4 * ks + gq;
        const bf16x8 a = *(const bf16x8*)(R + row * DR + 8 * (c ^ (row & (SR - 1))));
        sh[t] = mfma16(a, qh[KL + ks], sh[t]);
        sl[t] = mfma16(a, ql[KL + ks], sl[t]);
      }
    }
    const int j0 = w0 + blk * DT;
    float s[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool ok = j0 + 16 * t + 4 * gq + i < w1;
        s[t][i] = ok ? sh[t][i] + sl[t][i] : -INFINITY;
        mt = fmaxf(mt, s[t][i]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (__builtin_amdgcn_ballot_w64(mt > m_ref + kTauD) != 0) {
      const float m_new = fmaxf(m_ref, mt);
      const float al = __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_lane *= al;
      // accumulator rows are heads 4 gq + i, whose state sits in lane 4 gq + i
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(al, 4 * gq + i);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ct][i] *= ar[i];
    }
    // P (A operand: row = head n, contraction slots 8 gq .. 8 gq + 7 = tokens
    // 4 gq + i of tile 0, then of tile 1) and its fp32 sum from the same bf16
    bf16x8 pf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16 e = (bf16)__builtin_amdgcn_exp2f(s[t][i] - m_ref);
        pf[4 * t + i] = e;
        l_lane += (float)e;
      }
    // X_lat operand of column tile ct, read transposed: this lane addresses
    // row 4 (lane >> 4) + ((lane >> 2) & 3) (+ 16 for the second read) at
    // columns 16 ct + 4 (lane & 3) .. + 3 and receives tokens 4 gq .. 4 gq + 3
    // (then 16 + ...) of column 16 ct + n.
    const int r = lane & 3, k = (lane >> 2) & 3;
    const int ra = 4 * gq + k, rb = 16 + 4 * gq + k;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = 2 * ct + (r >> 1), half = r & 1;
      const bf16* pa = L + ra * DD + 8 * (c ^ (ra & 15)) + 4 * half;
      const bf16* pb = L + rb * DD + 8 * (c ^ (rb & 15)) + 4 * half;
      const s16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)pa);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)pb);
      // whole dwords: tokens 4 gq .. 4 gq + 3 then 16 + 4 gq .. (element order kept)
      const u32x2 ua = __builtin_bit_cast(u32x2, va), ub = __builtin_bit_cast(u32x2, vb);
      const u32x4 uw = {ua[0], ua[1], ub[0], ub[1]};
      acc[ct] = mfma16(pf, __builtin_bit_cast(bf16x8, uw), acc[ct]);
    }
  };

  // Block k lives in buffer k % NB; loads run NB - 1 blocks ahead.  Before
  // block blk is read, every load but those of the (up to NB - 2) blocks
  // issued after it must have landed.
  for (int k = 0; k < NB - 1 && k < nblk; ++k) issue(k, k);
  for (int blk = 0; blk < nblk; ++blk) {
    __asm__ volatile("" ::: "memory");
    if (blk + NB - 1 < nblk) issue(blk + NB - 1, (blk + NB - 1) % NB);
    const int ahead = min(nblk - 1 - blk, NB - 1);
    if constexpr (NB >= 3) {
      if (ahead >= 2) wait_vm<2 * (NL + NR)>();
      else if (ahead == 1) wait_vm<NL + NR>();
      else wait_vm<0>();
    } else {
      if (ahead == 1) wait_vm<NL + NR>();
      else wait_vm<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    __asm__ volatile("" ::: "memory");
    compute(blk, blk % NB);
  }

  // Merge the two waves' partials (wave 1 -> LDS -> wave 0), then write one
  // (max, sum, accumulator) per head of the group.
  float l_head = l_lane + __shfl_xor(l_lane, 16);
  l_head += __shfl_xor(l_head, 32);
  __asm__ volatile("" ::: "memory");
  __syncthreads();  // every wave is done with its staging buffers
  float* xacc = (float*)&sm.lat[1][0][0];  // [16 heads][DD]
  float* xml = (float*)&sm.lat[1][1][0];   // [2][16]
  if (wave == 1) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) xacc[(4 * gq + i) * DD + 16 * ct + n] = acc[ct][i];
    if (gq == 0) {
      xml[n] = m_ref;
      xml[16 + n] = l_head;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const float m1 = xml[n], l1 = xml[16 + n];
    const float M = fmaxf(l_head > 0.f ? m_ref : -INFINITY, l1 > 0.f ? m1 : -INFINITY);
    const float f0 = l_head > 0.f ? __builtin_amdgcn_exp2f(m_ref - M) : 0.f;
    const float f1 = l1 > 0.f ? __builtin_amdgcn_exp2f(m1 - M) : 0.f;
    const float L = f0 * l_head + f1 * l1;
    float g0[4], g1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      g0[i] = __shfl(f0, 4 * gq + i);
      g1[i] = __shfl(f1, 4 * gq + i);
    }
    const size_t PF = 2 + (size_t)DD;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int head = hg * 16 + 4 * gq + i;
      if (head < p.H) {
        float* dst = part + (((size_t)b * p.H + head) * g.n_chunks + chunk) * PF + 2;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          dst[16 * ct + n] = g0[i] * acc[ct][i] + g1[i] * xacc[(4 * gq + i) * DD + 16 * ct + n];
      }
    }
    const int head = hg * 16 + n;
    if (gq == 0 && head < p.H) {
      float* dst = part + (((size_t)b * p.H + head) * g.n_chunks + chunk) * PF;
      dst[0] = L > 0.f ? M : kNegBigD;
      dst[1] = L;
    }
  }
}

// Window part: the positions p-w+1 .. p of (batch, head).  A key's content
// row (2 d_k bytes) is read by d_k/8 lanes, 16 bytes each, its rotary row by
// the first d_R/8 of them; the lanes' partial dot products meet by shuffles.
// Keys go in tiles of up to WT: scores into LDS, the tile's maximum and
// exponentials, then the values read the same way, each lane accumulating
// its 8 columns; the key groups' accumulators are summed through LDS at the end.
template <int D, int DR>
__device__ __forceinline__ void window_block(const DropeDecodeProblem& p, const DropeGeom& g,
                                             float* part_win, int blk) {
  constexpr int LPK = D / 8, KPI = 256 / LPK, RL = DR / 8, WT = 1024;
  __shared__ float sc[WT];
  __shared__ float red[2][4];
  __shared__ float accs[KPI][D];
  const int bh = blk / g.n_win, piece = blk % g.n_win, b = bh / p.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = tid % LPK, kg = tid / LPK;
  const long pp = (long)p.ctx - 1;
  const long lw = pp - p.w + 1 > 0 ? pp - p.w + 1 : 0;  // first window position
  const int nw_all = p.w > 0 ? (int)(pp - lw + 1) : 0;
  // this piece: window positions lo .. lo + nw - 1
  const int k_begin = min(nw_all, piece * g.win_len);
  const long lo = lw + k_begin;
  const int nw = min(nw_all, k_begin + g.win_len) - k_begin;
  const float scl = kLog2e / sqrtf((float)(D + DR));
  float qc[8], qr[8];
  {
    const bf16x8 v = *(const bf16x8*)((const bf16*)p.qC + (size_t)bh * D + 8 * lr);
#pragma unroll
    for (int e = 0; e < 8; ++e) qc[e] = (float)v[e] * scl;
    if (lr < RL) {
      const bf16x8 u = *(const bf16x8*)((const bf16*)p.qR + (size_t)bh * DR + 8 * lr);
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[e] = (float)u[e] * scl;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qr[e] = 0.f;
    }
  }
  const bf16* Kw = (const bf16*)p.K_win + (size_t)bh * p.w * D;
  const bf16* Vw = (const bf16*)p.V_win + (size_t)bh * p.w * D;
  const bf16* Kr = (const bf16*)p.KR + (size_t)b * p.cap * DR;
  auto block_max = [&](float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
    if (lane == 0) red[0][wave] = x;
    __syncthreads();
    x = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    return x;
  };
  auto block_sum = [&](float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if (lane == 0) red[1][wave] = x;
    __syncthreads();
    return red[1][0] + red[1][1] + red[1][2] + red[1][3];
  };
  float m = kNegBigD, l = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int k0 = 0; k0 < nw; k0 += WT) {
    const int nt = min(WT, nw - k0);
#pragma unroll 8
    for (int kk = kg; kk < nt; kk += KPI) {
      const long j = lo + k0 + kk;
      const bf16x8 v = *(const bf16x8*)(Kw + (size_t)(j % p.w) * D + 8 * lr);
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf((float)v[e], qc[e], a);
      if (lr < RL) {
        const bf16x8 u = *(const bf16x8*)(Kr + (size_t)j * DR + 8 * lr);
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaf((float)u[e], qr[e], a);
      }
#pragma unroll
      for (int off = LPK / 2; off >= 1; off >>= 1) a += __shfl_xor(a, off);
      if (lr == 0) sc[kk] = a;
    }
    __syncthreads();
    float mt = -INFINITY;
    for (int kk = tid; kk < nt; kk += 256) mt = fmaxf(mt, sc[kk]);
    mt = block_max(mt);
    const float m_new = fmaxf(m, mt);
    const float al = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float ls = 0.f;
    for (int kk = tid; kk < nt; kk += 256) {
      const float e = __builtin_amdgcn_exp2f(sc[kk] - m);
      sc[kk] = e;
      ls += e;
    }
    ls = block_sum(ls);  // its barrier also publishes the exponentials
    l = l * al + ls;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= al;
#pragma unroll 8
    for (int kk = kg; kk < nt; kk += KPI) {
      const long j = lo + k0 + kk;
      const bf16x8 v = *(const bf16x8*)(Vw + (size_t)(j % p.w) * D + 8 * lr);
      const float pk = sc[kk];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(pk, (float)v[e], acc[e]);
    }
    __syncthreads();  // sc and red are rewritten by the next tile
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) accs[kg][8 * lr + e] = acc[e];
  __syncthreads();
  float* dst = part_win + ((size_t)bh * g.n_win + piece) * (2 + D);
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < KPI; ++k) a += accs[k][tid];
    dst[2 + tid] = a;
  }
  if (tid == 0) {
    dst[0] = nw > 0 ? m : -INFINITY;
    dst[1] = l;
  }
}

// One launch for both: the window needs no absorbed query, so the absorb
// blocks (dispatched first) finish under the window pieces' loads instead of
// as a latency-bound launch of their own.
template <int D, int DR>
__global__ __launch_bounds__(256) void drope_absorb_window(DropeDecodeProblem p, DropeGeom g,
                                                           bf16* qa_hi, bf16* qa_lo,
                                                           float* part_win, int n_abs) {
  const int bid = blockIdx.x;
  if (bid < n_abs) {
    const int ny = (g.qw + 63) / 64;
    absorb_block<D, DR>(p, g, qa_hi, qa_lo, bid % p.H, (bid / p.H) % ny, bid / (p.H * ny));
  } else {
    window_block<D, DR>(p, g, part_win, bid - n_abs);
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

bool drope_decode_supported(int d_k, int d_R, int d_down) {
  return (d_k == 64 || d_k == 128) && d_R == 64 &&
         (d_down == 128 || d_down == 256 || d_down == 512);
}

size_t drope_decode_workspace_bytes(const DropeDecodeProblem& p) {
  const DropeGeom g = drope_geom(p);
  const size_t qa = align256(sizeof(bf16) * (size_t)p.B * p.H * g.qw);
  const size_t lat = align256(sizeof(float) * (size_t)p.B * p.H * g.n_chunks * (2 + p.d_down));
  const size_t win = align256(sizeof(float) * (size_t)p.B * p.H * g.n_win * (2 + p.d_k));
  return 2 * qa + lat + win;
}

hipError_t launch_attn_decode_drope(const DropeDecodeProblem& p, hipStream_t s) {
  const DropeGeom g = drope_geom(p);
  char* ws = (char*)p.ws;
  const size_t qa = align256(sizeof(bf16) * (size_t)p.B * p.H * g.qw);
  const size_t lat = align256(sizeof(float) * (size_t)p.B * p.H * g.n_chunks * (2 + p.d_down));
  bf16* qa_hi = (bf16*)ws;
  bf16* qa_lo = (bf16*)(ws + qa);
  float* part_lat = (float*)(ws + 2 * qa);
  float* part_win = (float*)(ws + 2 * qa + lat);
  const int n_abs = p.H * ((g.qw + 63) / 64) * ((p.B + 3) / 4);
  const dim3 gaw(n_abs + p.B * p.H * g.n_win);
  const int n_stream = p.B * g.n_hg * g.n_chunks;
  if (p.d_k == 64) {
    hipLaunchKernelGGL((drope_absorb_window<64, 64>), gaw, dim3(256), 0, s, p, g, qa_hi, qa_lo,
                       part_win, n_abs);
    if (p.d_down == 128)
      hipLaunchKernelGGL((drope_stream<64, 128, 64, kStreamNB>), dim3(n_stream), dim3(DWAVES * 64),
                         0, s, p, g, qa_hi, qa_lo, part_lat);
    else if (p.d_down == 256)
      hipLaunchKernelGGL((drope_stream<64, 256, 64, kStreamNB>), dim3(n_stream), dim3(DWAVES * 64),
                         0, s, p, g, qa_hi, qa_lo, part_lat);
    else
      hipLaunchKernelGGL((drope_stream<64, 512, 64, 2>), dim3(n_stream), dim3(DWAVES * 64), 0, s,
                         p, g, qa_hi, qa_lo, part_lat);
  } else {
    hipLaunchKernelGGL((drope_absorb_window<128, 64>), gaw, dim3(256), 0, s, p, g, qa_hi, qa_lo,
                       part_win, n_abs);
    if (p.d_down == 128)
      hipLaunchKernelGGL((drope_stream<128, 128, 64, kStreamNB>), dim3(n_stream),
                         dim3(DWAVES * 64), 0, s, p, g, qa_hi, qa_lo, part_lat);
    else if (p.d_down == 256)
      hipLaunchKernelGGL((drope_stream<128, 256, 64, kStreamNB>), dim3(n_stream),
                         dim3(DWAVES * 64), 0, s, p, g, qa_hi, qa_lo, part_lat);
    else
      hipLaunchKernelGGL((drope_stream<128, 512, 64, 2>), dim3(n_stream), dim3(DWAVES * 64), 0, s,
                         p, g, qa_hi, qa_lo, part_lat);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeProblem c{};
  c.W_upV = p.W_upV;
  c.o = p.o;
  c.B = p.B;
  c.H = p.H;
  c.d_k = p.d_k;
  c.d_down = p.d_down;
  return launch_decode_combine(c, g.n_chunks, part_lat, part_win, g.n_win, s);
}

}  // namespace dar
