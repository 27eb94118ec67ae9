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
// bf16 mode: workgroup tiles of 256 tokens x 128 columns, 4 waves of 128x64
// built from 32x32x16 MFMAs, k-tiles of 32 in a 3-stage LDS ring filled by
// direct global-to-LDS buffer loads, fp32 accumulate, epilogue staged through
// LDS so the rotate-half partners (t, t + d_k/2) meet in one thread and stores
// coalesce.
// The projections are written as IEEE fp16 (3 more mantissa bits than bf16 at
// the same size and MFMA rate); the second GEMM therefore runs on fp16 MFMAs,
// converting the bf16 folded weights to fp16 as they are staged into LDS.
// fp32 path: an LDS-tiled VALU GEMM with the same epilogue (no bf16 anywhere).
#include <type_traits>

#include "dar_common.hpp"

namespace dar {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDA_S = BK + 8;  // bf16 per LDS row: 144 B, rows land 4 banks apart
constexpr int EPI_P = BN + 4;  // fp32 per epilogue row
#ifndef DAR_WIDE_MIN_TILES
#define DAR_WIDE_MIN_TILES 512
#endif
// wide-tile GEMM from this many tiles (two per CU; the Pythia-410M-shaped
// first GEMM, 832 tiles, gains 5.5% over the 256 x 128 kernel)
constexpr long kWideMinTiles = DAR_WIDE_MIN_TILES;
#ifndef DAR_WIDE_BAND_BYTES
#define DAR_WIDE_BAND_BYTES (4 << 20)
#endif
constexpr long kWideBandBytes = DAR_WIDE_BAND_BYTES;  // weight bytes of one band
// The wide kernel's one workgroup per CU cannot overlap the epilogue with
// another tile's main loop, which a long main loop amortizes: bf16
// activations need K >= 1024 (the first projection GEMM).  The fp16 global
// GEMM (K = d_down = 512 at the 1B scale) gains 1.4% of the projection with
// the eight-wave kernel and its split stores.
constexpr int kWideMinK = 1024;

// Slot of k-chunk c (of 4 per 64-byte row) in row r of a staged k-tile:
// c ^ kswz(r).  Any 16 consecutive rows read at one chunk index then cover
// all 64 banks once, which is what the 16-byte fragment reads need (measured:
// a swizzle built for 8-lane groups over 32 banks raised the bank-conflict
// cycles of the GEMM from 2% to 12% of its run time).
__device__ __forceinline__ int kswz(int r) { return (r >> 2) & 3; }

struct SegTiles {
  int tile0[5];  // first column tile of each segment, tile0[nseg] = total
};

__device__ __forceinline__ int find_seg(const SegTiles& st, int nseg, int ct) {
  int s = 0;
  while (s + 1 < nseg && ct >= st.tile0[s + 1]) ++s;
  return s;
}

// Stores n consecutive fp32 values as OutT with the widest aligned stores.
template <typename OutT, int NV>
__device__ __forceinline__ void store_run(OutT* dst, const float* v) {
  if constexpr (sizeof(OutT) == 2) {
    static_assert(NV % 8 == 0, "fp16 runs are stored 8 at a time");
#pragma unroll
    for (int i = 0; i < NV; i += 8) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = __is_same(OutT, f16) ? pack_f16x2(v[i + 2 * e], v[i + 2 * e + 1])
                                    : pack_bf16x2(v[i + 2 * e], v[i + 2 * e + 1]);
      // streaming stores: the outputs are read by the next kernels, not
      // here, so they should not push the tiles this kernel reuses out of L2
      __builtin_nontemporal_store(w, (u32x4*)(dst + i));
    }
  } else {
    static_assert(NV % 4 == 0, "fp32 runs are stored 4 at a time");
#pragma unroll
    for (int i = 0; i < NV; i += 4) {
      const f32x4 x = {v[i], v[i + 1], v[i + 2], v[i + 3]};
      __builtin_nontemporal_store(x, (f32x4*)(dst + i));
    }
  }
}

// Four consecutive fp32 values as OutT (8 or 16 bytes).
template <typename OutT>
__device__ __forceinline__ void store_run4(OutT* dst, const float* v) {
  if constexpr (sizeof(OutT) == 2) {
    u32x2 w;
    w[0] = __is_same(OutT, f16) ? pack_f16x2(v[0], v[1]) : pack_bf16x2(v[0], v[1]);
    w[1] = __is_same(OutT, f16) ? pack_f16x2(v[2], v[3]) : pack_bf16x2(v[2], v[3]);
    *(u32x2*)dst = w;
  } else {
    *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Writes a [ROWS x BN] fp32 tile held in LDS (pitch EPI_P) to segment `seg`.
// Tile row r is GEMM row row0 + r, i.e. token (b, n) = divmod(row0 + r, n_seq);
// tile column c is segment column col0 + c.  Each thread owns one row and a
// contiguous run of columns (kHeadT: one column and a run of rows), so the
// (b, n) division happens once per thread and stores are 8-16 bytes wide.
// Logistic sigmoid 1 / (1 + e^-x) in fp32, for the variant that applies it
// after the down-projection of Eq. (1): e^-x as 2^(-x log2 e) and the
// hardware reciprocal (a few ulp; the latent is then rounded to 16 bits in
// bf16 mode).  Large negative x gives 2^+inf = inf and 0, large positive 1.
__device__ __forceinline__ void sigmoid8(float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-v[e] * kLog2e));
}

template <typename OutT, int D, int ROWS>
__device__ void epilogue_store(const float* tile, int row0, int col0, const GemmSeg& seg,
                               const GemmProblem& p) {
  constexpr int TPR = 256 / ROWS;  // threads per tile row
  constexpr int CPT = BN / TPR;    // columns per thread
  const int tid = threadIdx.x;
  const int M = p.M, width = seg.width, H = seg.heads ? seg.heads : p.heads, Nq = p.n_seq;
  OutT* out = (OutT*)seg.out;
  if (seg.kind == kHeadT) {
    // out[b, head, t, n]: thread = (column c, run of ROWS/2 rows)
    constexpr int RPT = ROWS / 2;
    const int c = tid % BN, r0 = (tid / BN) * RPT;
    const int gcol = col0 + c;
    if (gcol >= width) return;
    const int head = gcol / D, t = gcol % D;
    const int grow0 = row0 + r0;
    const int ld = seg.ld_seq ? seg.ld_seq : Nq;
    const int b0 = grow0 / Nq, n0 = grow0 % Nq, no0 = n0 + seg.seq_off;
    float v[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) v[i] = tile[(r0 + i) * EPI_P + c];
    const bool fast =
        (grow0 + RPT <= M) && (n0 + RPT <= Nq) && ((no0 & 7) == 0) && ((ld & 7) == 0);
    if (fast) {
      store_run<OutT, RPT>(out + (((size_t)b0 * H + head) * D + t) * ld + no0, v);
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int grow = grow0 + i;
        if (grow >= M) break;
        const int b = grow / Nq, n = grow % Nq;
        out[(((size_t)b * H + head) * D + t) * ld + n + seg.seq_off] = from_f32<OutT>(v[i]);
      }
    }
    return;
  }
  const int r = tid / TPR, part = tid % TPR;
  const int grow = row0 + r;
  if (grow >= M) return;
  const int b = grow / Nq, n = grow % Nq;
  const int ld = seg.ld_seq ? seg.ld_seq : Nq;  // output sequence stride
  const int no = n + seg.seq_off;                // output sequence index
  const float* trow = tile + r * EPI_P;
  if (seg.kind == kRowMajor) {
    // width is a multiple of 32: the run is stored in chunks of 8 columns,
    // each either wholly inside the segment or wholly past its end
    const int c = part * CPT;
    OutT* dst = out + ((size_t)b * ld + no) * width + col0 + c;
#pragma unroll
    for (int i = 0; i < CPT; i += 8) {
      if (col0 + c + i >= width) break;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = trow[c + i + e];
      if (seg.act) sigmoid8(v);
      store_run<OutT, 8>(dst + i, v);
    }
    return;
  }
  // kHead: out[b, head, n, t]
  if (!seg.rope) {
    const int c = part * CPT;
    const int gcol = col0 + c;
    if (gcol >= width) return;
    const int head = gcol / D, t = gcol % D;  // CPT divides D: the run stays in one head
    float v[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) v[i] = trow[c + i];
    store_run<OutT, CPT>(out + (((size_t)b * H + head) * ld + no) * D + t, v);
    return;
  }
  // RoPE at position pos0 + n on rotate-half pairs (t, t + D/2): the thread
  // takes CPT/2 consecutive pairs of one head.
  constexpr int HALF = D / 2, PPT = CPT / 2;
  const int q0 = part * PPT;              // first pair of this thread within the tile
  const int hl = q0 / HALF, t0 = q0 % HALF;
  const int gcol = col0 + hl * D;
  if (gcol >= width) return;
  const int head = gcol / D;
  const int pos = p.pos0 + n;
  const float* x = trow + hl * D + t0;
  const float* y = x + HALF;
  float a[PPT], bb[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const float2 cs = rope_cs(p.rope, pos, t0 + i);
    a[i] = x[i] * cs.x - y[i] * cs.y;
    bb[i] = x[i] * cs.y + y[i] * cs.x;
  }
  OutT* dst = out + (((size_t)b * H + head) * ld + no) * D + t0;
  store_run<OutT, PPT>(dst, a);
  store_run<OutT, PPT>(dst + HALF, bb);
}

// --------------------------------------------------------------------------
// Stores of the MFMA GEMM epilogue.  One epilogue pass holds 128 tokens of the
// workgroup tile in LDS: tile row r is GEMM row epi_row(row0, hf, r) (the two
// 64-token runs starting at 64 hf and 128 + 64 hf).  Work is cut into 16-byte
// output chunks (8 values) so that eight consecutive lanes write 128
// contiguous bytes, and the lane order keeps the LDS reads conflict-free.
// RoPE position of token (b, n), and its index in the output sequence of
// segment seg (stride ld): fixed offsets, or per-row positions of a ragged
// append (one token per sequence).
// RP (compile time): the problem carries row_pos.
template <bool RP>
__device__ __forceinline__ int row_position(const GemmProblem& p, int b, int n) {
  if constexpr (!RP) {
    const int q = p.pos0 + n;  // ragged rows: clamped into the tables
    return p.cu != nullptr ? min(max(q, 0), p.pos_max) : q;
  }
  const int q = p.row_pos[b];
  return q < 0 ? 0 : (q > p.pos_max ? p.pos_max : q);
}

template <bool RP>
__device__ __forceinline__ int out_index(const GemmProblem& p, const GemmSeg& seg, int b, int n,
                                         int ld) {
  if constexpr (!RP) return n + seg.seq_off;
  if (seg.pos_mode == kPosFixed) return n + seg.seq_off;
  const int q = row_position<RP>(p, b, n);
  return seg.pos_mode == kPosRing ? q % ld : min(q, ld - 1);
}

// Where GEMM row `grow` goes: its sequence b, its index n and the sequence's
// length, and the output's row base and sequence stride.  Head-major outputs
// put token n of head `head` at row base * H + head * ld + n (V: column
// base * H * D + (head * D + t) * ld + n); row-major ones at row base + n.
// Uniform sequences: base = b * ld.  Ragged (cu): one block per sequence at
// its first row, the sequence's row range clamped into [0, M]; `ok` is false
// for a row outside the range found (inconsistent cu), which is not written.
// Row of A read by GEMM row g: g itself, or with a_ld_seq set, row n of
// sequence b = g / n_seq at b a_ld_seq + n.
__device__ __forceinline__ int a_row(const GemmProblem& p, int g) {
  return p.a_ld_seq > 0 ? (g / p.n_seq) * p.a_ld_seq + g % p.n_seq : g;
}

struct RowLoc {
  int b, n, len, ld;
  size_t base;
  bool ok;
};

__device__ __forceinline__ RowLoc row_loc(const GemmProblem& p, const GemmSeg& seg, int grow) {
  RowLoc r;
  if (p.cu != nullptr) {
    int lo = 0, hi = p.n_cu;  // the last b with cu[b] <= grow
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu[mid] <= grow) lo = mid; else hi = mid;
    }
    const int c0 = min(max(p.cu[lo], 0), p.M), c1 = min(max(p.cu[lo + 1], c0), p.M);
    r.b = lo;
    r.n = grow - c0;
    r.len = c1 - c0;
    r.ld = r.len;
    r.base = (size_t)c0;
    r.ok = r.n >= 0 && r.n < r.len;
  } else {
    const int Nq = p.n_seq;
    r.b = grow / Nq;
    r.n = grow % Nq;
    r.len = Nq;
    r.ld = seg.ld_seq ? seg.ld_seq : Nq;
    r.base = (size_t)r.b * r.ld;
    r.ok = true;
  }
  return r;
}

// RoPE position of row n of a sequence (ragged rows clamped into the tables).
__device__ __forceinline__ int seq_position(const GemmProblem& p, int n) {
  const int q = p.pos0 + n;
  return p.cu != nullptr ? min(max(q, 0), p.pos_max) : q;
}

__device__ __forceinline__ int epi_row(int row0, int hf, int r) {
  return row0 + 128 * (r >> 6) + 64 * hf + (r & 63);
}

__device__ __forceinline__ void read8(const float* src, float (&v)[8]) {
  const float4 a = *(const float4*)src, b = *(const float4*)(src + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// cos/sin(pos * theta_t) for t = t0 .. t0+7 from the two-level tables.
__device__ __forceinline__ void rope_cs8(const RopeTab& t, int pos, int t0, float2 (&cs)[8]) {
  const float4* hi = (const float4*)(t.hi + (size_t)(pos >> 6) * t.half + t0);
  const float4* lo = (const float4*)(t.lo + (size_t)(pos & 63) * t.half + t0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = hi[i], b = lo[i];
    cs[2 * i] = make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
    cs[2 * i + 1] = make_float2(a.z * b.z - a.w * b.w, a.z * b.w + a.w * b.z);
  }
}

// Tile [128 tokens][PITCH] (128 columns used) -> kRowMajor, or kHead without rotation.
template <typename OutT, int D, bool RP, int PITCH = EPI_P>
__device__ __forceinline__ void store_rows_plain(const float* tile, int row0, int hf, int col0,
                                                 const GemmSeg& seg, const GemmProblem& p,
                                                 int tid = threadIdx.x) {
  const int M = p.M, width = seg.width, H = seg.heads ? seg.heads : p.heads;
  OutT* out = (OutT*)seg.out;
  // chunk q = tid + 256 k: column chunk (q & 7) + 8 (q >> 10), tile row (q >> 3) & 127;
  // chunks k and k + 4 share the row
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = ((tid >> 3) + 32 * k) & 127;
    const int grow = epi_row(row0, hf, r);
    if (grow >= M) continue;
    const RowLoc L = row_loc(p, seg, grow);
    if (!L.ok) continue;
    const int no = out_index<RP>(p, seg, L.b, L.n, L.ld);
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c = 8 * ((tid & 7) + 8 * h2);
      const int gcol = col0 + c;  // width is a multiple of 32: chunks are whole
      if (gcol >= width) continue;
      float v[8];
      read8(tile + r * PITCH + c, v);
      OutT* dst;
      if (seg.kind == kRowMajor) {
        dst = out + (L.base + no) * width + gcol;
        if (seg.act) sigmoid8(v);
      } else {
        const int head = gcol / D, t = gcol % D;
        dst = out + (L.base * H + (size_t)head * L.ld + no) * D + t;
      }
      store_run<OutT, 8>(dst, v);
    }
  }
}

// Tile [128 tokens][PITCH] (128 columns used) -> kHead with RoPE at position pos0 + n on the
// rotate-half pairs (t, t + D/2).  A lane takes 8 consecutive pairs of one head
// for 4 consecutive tokens: the angles of the first token come from the
// tables, the next ones by one complex multiplication with (cos, sin)(theta_t)
// each (the table row for position 1).
// cos/sin of the first of the 4 tokens a thread of store_rows_rope takes in
// epilogue pass hf, for its 8 pairs, and the one-position step; loaded ahead
// (at kernel start) so their latency hides under the main loop.
struct RopePre {
  float2 cs[8], step[8];
};

template <int D>
__device__ __forceinline__ void rope_prefetch(const GemmProblem& p, int row0, int hf,
                                              RopePre& r) {
  constexpr int PCH = D / 16;
  const int tid = threadIdx.x, w8 = tid & 7, t0 = 8 * (w8 % PCH);
  const int grow0 = epi_row(row0, hf, 4 * (tid >> 3));
  GemmSeg none{};
  const RowLoc L = row_loc(p, none, grow0 < p.M ? grow0 : 0);
  rope_cs8(p.rope, seq_position(p, L.ok ? L.n : 0), t0, r.cs);
  const float4* st = (const float4*)(p.rope.lo + p.rope.half + t0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 a = st[i];
    r.step[2 * i] = make_float2(a.x, a.y);
    r.step[2 * i + 1] = make_float2(a.z, a.w);
  }
}

template <typename OutT, int D, bool RP, int PITCH = EPI_P>
__device__ __forceinline__ void store_rows_rope(const float* tile, int row0, int hf, int col0,
                                                const GemmSeg& seg, const GemmProblem& p,
                                                const RopePre* pre = nullptr,
                                                int tid = threadIdx.x) {
  constexpr int HALF = D / 2, PCH = D / 16;  // pair chunks of 8 per head
  const int M = p.M, width = seg.width, H = seg.heads ? seg.heads : p.heads;
  OutT* out = (OutT*)seg.out;
  const int w8 = tid & 7, r0 = 4 * (tid >> 3);
  const int hl = w8 / PCH, t0 = 8 * (w8 % PCH);
  const int c = hl * D + t0;  // tile column of x; y sits HALF further
  const int gcol = col0 + hl * D;
  const int grow0 = epi_row(row0, hf, r0);
  if (gcol >= width || grow0 >= M) return;
  const int head = gcol / D;
  const RowLoc L0 = row_loc(p, seg, grow0);
  // one sequence, consecutive positions
  const bool consec = L0.ok && grow0 + 3 < M && L0.n + 3 < L0.len;
  float2 cs[8], step[8];
  if (!RP && pre != nullptr && consec) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cs[i] = pre->cs[i];
      step[i] = pre->step[i];
    }
  } else {
    rope_cs8(p.rope, row_position<RP>(p, L0.b, L0.n), t0, cs);
    if (consec) {
      const float4* st = (const float4*)(p.rope.lo + p.rope.half + t0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 a = st[i];
        step[2 * i] = make_float2(a.x, a.y);
        step[2 * i + 1] = make_float2(a.z, a.w);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    RowLoc L = L0;
    L.n += kk;
    if (kk > 0) {
      if (consec) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          cs[i] = make_float2(cs[i].x * step[i].x - cs[i].y * step[i].y,
                              cs[i].x * step[i].y + cs[i].y * step[i].x);
      } else {
        const int grow = grow0 + kk;
        if (grow >= M) break;
        L = row_loc(p, seg, grow);
        rope_cs8(p.rope, row_position<RP>(p, L.b, L.n), t0, cs);
      }
    }
    if (!L.ok) continue;
    float x[8], y[8], a[8], bb[8];
    read8(tile + (r0 + kk) * PITCH + c, x);
    read8(tile + (r0 + kk) * PITCH + c + HALF, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = x[i] * cs[i].x - y[i] * cs[i].y;
      bb[i] = x[i] * cs[i].y + y[i] * cs[i].x;
    }
    OutT* dst =
        out + (L.base * H + (size_t)head * L.ld + out_index<RP>(p, seg, L.b, L.n, L.ld)) * D + t0;
    store_run<OutT, 8>(dst, a);
    store_run<OutT, 8>(dst + HALF, bb);
  }
}

// Tile [128 columns][TP] (token innermost) -> kHeadT, out[b, head, t, n].
template <typename OutT, int D, int TP>
__device__ __forceinline__ void store_cols(const float* tile, int row0, int hf, int col0,
                                           const GemmSeg& seg, const GemmProblem& p,
                                           int tid = threadIdx.x) {
  const int M = p.M, width = seg.width, H = seg.heads ? seg.heads : p.heads;
  OutT* out = (OutT*)seg.out;
  const int tc = tid & 7;  // chunk of 8 tokens within the 64-token run
#pragma unroll
  for (int run = 0; run < 2; ++run) {
    const int grow0 = row0 + 128 * run + 64 * hf + 8 * tc;
    if (grow0 >= M) continue;
    const RowLoc L0 = row_loc(p, seg, grow0);
    const int no0 = L0.n + seg.seq_off;
    // the 8 tokens in one sequence: one address; 16-byte aligned runs store whole
    const bool same = L0.ok && (grow0 + 8 <= M) && (L0.n + 8 <= L0.len);
    const bool fast = same && ((no0 & 7) == 0) && ((L0.ld & 7) == 0);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = (tid >> 3) + 32 * k;
      const int gcol = col0 + c;
      if (gcol >= width) continue;
      const int head = gcol / D, t = gcol % D;
      float v[8];
      read8(tile + c * TP + 64 * run + 8 * tc, v);
      OutT* dst = out + L0.base * H * D + ((size_t)head * D + t) * L0.ld + no0;
      if (fast) {
        store_run<OutT, 8>(dst, v);
      } else if (same) {
#pragma unroll
        for (int i = 0; i < 8; ++i) dst[i] = from_f32<OutT>(v[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int grow = grow0 + i;
          if (grow >= M) break;
          const RowLoc L = row_loc(p, seg, grow);
          if (!L.ok) continue;
          out[L.base * H * D + ((size_t)head * D + t) * L.ld + L.n + seg.seq_off] =
              from_f32<OutT>(v[i]);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// MFMA GEMM: A and the MFMA operands of type TM (bf16 or fp16), B stored as TB
// (converted to TM while staged), outputs of type TO.
//
// The MFMA computes the transposed tile C^T = B^T A^T: the weight rows (output
// columns) are the first operand and the token rows the second, so a lane's
// accumulators hold one token and runs of 4 consecutive output columns, which
// go to an LDS staging tile as 16-byte writes ([token][column] for Q, K and h^D,
// [column][token] for the transposed V layout [b, head, t, n]).
template <typename TM, typename TB, typename TO, int D, bool RP>
__global__ __launch_bounds__(256, 2) void project_gemm_mfma(GemmProblem p, SegTiles st, int nM,
                                                           int nC, int nCp, int order) {
  typedef typename Vec8<TM>::type TMx8;
  typedef typename Vec8<TB>::type TBx8;
  // Workgroup tile: 256 tokens x 128 output columns; wave tile 128 tokens x 64
  // columns (two 32-column blocks that are rotate-half partners), so each
  // 16-wide k-step reads 6 fragments from LDS for 8 MFMAs.
  // Main loop: k-tiles of GBK = 32 in a 3-stage LDS ring filled by direct
  // buffer loads (global -> LDS, no staging registers; lanes past the matrix
  // edge read zeros), prefetching two k-tiles ahead, one barrier per k-tile.
  // Rows of a k-tile are 64 B = 4 chunks of 16 B; chunk c of row r sits in
  // slot c ^ kswz(r), which keeps the 16-byte MFMA fragment reads free of
  // bank conflicts.
  constexpr int TBM = 2 * BM;  // tokens per workgroup tile
  constexpr int GBK = 32, NST = 3;
  constexpr int TOK = TBM * GBK, STAGE = TOK + BN * GBK;  // elements per stage
  constexpr int MAIN_BYTES = NST * STAGE * 2, EPI_BYTES = BM * EPI_P * 4;
  __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES];
  // XCD-aware order.  order 0 (large weights): XCD x owns a contiguous group of
  // column tiles, whose slice of the weights stays in its L2, and walks the row
  // tiles in order.  order 1 (weights that fit in one L2): XCD x owns the row
  // tiles congruent to x and walks every column tile of one row tile before
  // the next, so each tile of activations is fetched once overall.
  const int bid = blockIdx.x;
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  int mt, ct;
  if (order == 0) {
    const int g = nCp / kNumXcd;
    mt = k / g;
    ct = x * g + (k % g);
  } else {
    mt = (k / nC) * kNumXcd + x;
    ct = k % nC;
  }
  if (ct >= nC || mt >= nM) return;
  const int s = find_seg(st, p.nseg, ct);
  const GemmSeg seg = p.seg[s];
  const int col0 = (ct - st.tile0[s]) * BN;  // first segment column of the tile
  const int row0 = mt * TBM;
  const int K = p.K, M = p.M;

  // the wave index is uniform: keep it in a scalar register so the LDS
  // destinations of the direct-to-LDS loads (M0) need no per-lane handling
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  // wave -> (partner pair of 32-column blocks, 128-token half)
  const int wp = wave & 1, wt = wave >> 1;
  const int cb0 = (D == 128) ? wp : 2 * wp;          // first column block (of 4)
  const int cb1 = (D == 128) ? wp + 2 : 2 * wp + 1;  // its rotate-half partner

  // Buffer resources over this tile's rows (byte extents; invalid lanes use an
  // offset past the extent and read zeros).
  const int ar0 = a_row(p, row0);
  const size_t a_ext = (size_t)(a_row(p, M - 1) + 1 - ar0) * K * sizeof(TM);
  const size_t b_ext = (size_t)(seg.width - col0) * K * sizeof(TB);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const TM*)p.A + (size_t)ar0 * K), (short)0,
      (int)(a_ext < 0x7ffffff0u ? a_ext : 0x7ffffff0u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const TB*)seg.Bt + (size_t)col0 * K), (short)0,
      (int)(b_ext < 0x7ffffff0u ? b_ext : 0x7ffffff0u), 0x00020000);
  TM* const lds = (TM*)smem;
  // One 16-byte chunk per lane per load: slot P of the k-tile holds chunk
  // (P & 3) ^ kswz(row) of row P >> 2.  K is a multiple of GBK, so
  // only rows can fall off the matrix; a lane's byte offset within a k-tile
  // is fixed (or past the buffer's extent, which reads zeros), and the
  // k-tile's offset goes in the scalar operand.
  unsigned va[4], vb[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = (i * 4 + wave) * 64 + lane, r = P >> 2;
    const int kc = 8 * ((P & 3) ^ kswz(r));
    va[i] = row0 + r < M ? (unsigned)(((a_row(p, row0 + r) - ar0) * K + kc) * sizeof(TM))
                         : 0x80000000u;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int P = (i * 4 + wave) * 64 + lane, r = P >> 2;
    const int kc = 8 * ((P & 3) ^ kswz(r));
    vb[i] = col0 + r < seg.width ? (unsigned)((r * K + kc) * sizeof(TB)) : 0x80000000u;
  }
  auto issue = [&](int kt, int stg) {
    const int ka = kt * GBK * (int)sizeof(TM), kb = kt * GBK * (int)sizeof(TB);
#pragma unroll
    for (int i = 0; i < 4; ++i)  // token rows: 1024 chunks
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(lds + stg * STAGE + (i * 4 + wave) * 512),
          16, va[i], ka, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i)  // weight rows: 512 chunks
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb,
          (__attribute__((address_space(3))) void*)(lds + stg * STAGE + TOK + (i * 4 + wave) * 512),
          16, vb[i], kb, 0, 0);
  };
  auto frag_off = [&](int row, int chunk) { return row * GBK + 8 * (chunk ^ kswz(row)); };

  // acc[i][j]: column block (cb0, cb1)[i] x token block j of this wave
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + GBK - 1) / GBK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    // this lane's loads of k-tile kt are done once at most those of kt+1 (6) remain
    if (kt + 1 < nk)
      __builtin_amdgcn_s_waitcnt(0x0F76);  // vmcnt(6)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    lds_barrier();  // k-tile kt is in LDS; everyone is done with k-tile kt-1
    if (kt + 2 < nk) issue(kt + 2, (kt + 2) % NST);
    const TM* sa = lds + (kt % NST) * STAGE;
    const TB* sb = (const TB*)(lds + (kt % NST) * STAGE + TOK);
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks) {
      const int ch = 2 * ks + lg;
      TMx8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = 32 * (i ? cb1 : cb0) + lr;
        const TBx8 w = *(const TBx8*)(sb + frag_off(row, ch));
        if constexpr (__is_same(TM, TB))
          a[i] = w;
        else
          a[i] = __builtin_bit_cast(TMx8, bf16x8_to_f16x8(__builtin_bit_cast(u32x4, w)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const TMx8*)(sa + frag_off(128 * wt + 32 * j + lr, ch));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  }

  // Epilogue in two passes through an LDS tile of 128 tokens.  Pass hf takes
  // token blocks j = 2hf, 2hf+1 of both wave halves, i.e. the two runs of 64
  // tokens starting at 64hf and 128 + 64hf; it frees half the accumulators.
  // Register r of acc[i][j] is column 32*cb_i + 8*(r/4) + 4*lg + r%4, token
  // 128*wt + 32*j + lr of the workgroup tile.
  float* tile = (float*)smem;
  // hf is a compile-time constant, so acc is only ever indexed statically
  auto pass = [&](auto HF) {
    constexpr int hf = decltype(HF)::value;
    // LDS free (main loop, or the previous pass's stores).  LDS order only: a
    // __syncthreads() would also wait for this wave's global stores.
    lds_barrier();
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * hf + jj;
      const int trow = 64 * wt + 32 * jj + lr;  // tile row of this lane's token
      if (seg.kind == kHeadT) {  // tile [column][token]
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 32 * (i ? cb1 : cb0) + 8 * (r >> 2) + 4 * lg + (r & 3);
            tile[c * (BM + 4) + trow] = acc[i][j][r];
          }
      } else {  // tile [token][column], float4 runs
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int c = 32 * (i ? cb1 : cb0) + 8 * a + 4 * lg;
            *(float4*)(tile + trow * EPI_P + c) =
                make_float4(acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2],
                            acc[i][j][4 * a + 3]);
          }
      }
    }
    lds_barrier();  // the tile is in LDS
    if (seg.kind == kHeadT)
      store_cols<TO, D, BM + 4>(tile, row0, hf, col0, seg, p);
    else if (seg.kind == kHead && seg.rope)
      store_rows_rope<TO, D, RP>(tile, row0, hf, col0, seg, p);
    else
      store_rows_plain<TO, D, RP>(tile, row0, hf, col0, seg, p);
  };
  pass(std::integral_constant<int, 0>{});
  pass(std::integral_constant<int, 1>{});
}

// --------------------------------------------------------------------------
// Wide MFMA GEMM for large problems: workgroup tiles of 256 tokens x 256
// output columns, one workgroup per CU.  Launched with 8 waves in a 4 x 2
// grid, each 128 tokens x 64 columns (8 accumulator blocks of 32 x 32), two
// waves per SIMD, so one wave's MFMAs cover the other's barrier and LDS
// waits; a 16-wide k-step reads 6 fragments from LDS for 8 MFMAs.  (With 4
// waves of 128 x 128, one per SIMD and 16 blocks each, a k-step reads 8
// fragments for 16 MFMAs but nothing covers a wave's stalls: 3% slower on
// the 1B-scale layer.)
//
// Tile order ("bands"): the column tiles are cut into bands of WB; a band's
// tiles are walked row tile by row tile, columns innermost, and the whole
// sequence (band after band) is cut into 8 equal contiguous parts, one per XCD
// (workgroup b runs on XCD b mod 8).  An XCD thus works on at most two bands
// at a time: their weights stay in its L2 while the activation rows stream,
// each read once per band; and every XCD gets the same number of tiles.
constexpr int WBN = 256;  // columns per wide tile

template <typename TM, typename TB, typename TO, int D, int GBK, int NW = 4>
__global__ __launch_bounds__(64 * NW, 1) void project_gemm_wide(GemmProblem p, SegTiles st,
                                                                int nM, int nC, int band,
                                                                int per_xcd) {
  typedef typename Vec8<TM>::type TMx8;
  typedef typename Vec8<TB>::type TBx8;
  constexpr int TBM = 256;
  // k-tiles of GBK (32 or 64) in an LDS ring of NST stages (4 x 32 KB or 2 x 64 KB)
  constexpr int NST = GBK == 64 ? 2 : 4;
  constexpr int CPR = GBK / 8;   // 16-byte chunks per staged row
  constexpr int KS = GBK / 16;   // MFMA k-steps per k-tile
  // NW = 4: a wave per SIMD, each 128 tokens x 128 columns; NW = 8: two per
  // SIMD, each 128 tokens x 64 columns (the other covers its stalls)
  static_assert(NW == 4 || NW == 8, "waves");
  constexpr int WCOLS = NW / 2, CW = WBN / WCOLS, NI = CW / 32;  // column groups, width, blocks
  constexpr int NLD = CPR * 4 / NW;  // loads per lane per operand per k-tile
  constexpr int LPT = 2 * NLD;   // direct-to-LDS loads per lane per k-tile
  static_assert(GBK == 32 || GBK == 64, "k-tile depth");
  constexpr int TOK = TBM * GBK, STAGE = TOK + WBN * GBK;  // elements per stage
  constexpr int RP_ = WBN + 4, CP_ = TBM / 2 + 4;           // epilogue pitches (fp32)
  constexpr int MAIN_BYTES = NST * STAGE * 2;
  constexpr int EPI_ROWS = 128 * RP_ * 4, EPI_COLS = WBN * CP_ * 4;
  constexpr int EPI_BYTES = EPI_ROWS > EPI_COLS ? EPI_ROWS : EPI_COLS;
  __shared__ __attribute__((aligned(16))) char smem[MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES];

  const int bid = blockIdx.x;
  const int seq = (bid % kNumXcd) * per_xcd + bid / kNumXcd;
  const int nfull = nC / band;  // bands of exactly `band` columns
  int mt, ct;
  if (seq < nfull * band * nM) {
    const int bd = seq / (band * nM), rem = seq % (band * nM);
    mt = rem / band;
    ct = bd * band + rem % band;
  } else {
    const int bw = nC - nfull * band, rem = seq - nfull * band * nM;
    if (bw == 0) return;
    mt = rem / bw;
    ct = nfull * band + rem % bw;
  }
  if (ct >= nC || mt >= nM) return;
  const int s = find_seg(st, p.nseg, ct);
  const GemmSeg seg = p.seg[s];
  const int col0 = (ct - st.tile0[s]) * WBN;
  const int row0 = mt * TBM;
  const int K = p.K, M = p.M;

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;
  const int wc = wave % WCOLS, wt = wave / WCOLS;  // column group, token half

  const int ar0 = a_row(p, row0);
  const size_t a_ext = (size_t)(a_row(p, M - 1) + 1 - ar0) * K * sizeof(TM);
  const size_t b_ext = (size_t)(seg.width - col0) * K * sizeof(TB);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const TM*)p.A + (size_t)ar0 * K), (short)0,
      (int)(a_ext < 0x7ffffff0u ? a_ext : 0x7ffffff0u), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const TB*)seg.Bt + (size_t)col0 * K), (short)0,
      (int)(b_ext < 0x7ffffff0u ? b_ext : 0x7ffffff0u), 0x00020000);
  TM* const lds = (TM*)smem;
  // 16-byte chunk P of a k-tile region: row P / CPR, slot P % CPR holding
  // k-chunk slot ^ swz(row) (32: kswz; 64: (row >> 1) & 7, which keeps 16
  // consecutive 128-byte rows read at one chunk on distinct banks).  As in
  // the 256 x 128 kernel, a lane's offset within a k-tile is fixed (rows past
  // the edge read zeros) and the k-tile's offset is the scalar operand.
  auto swz = [](int r) { return GBK == 64 ? (r >> 1) & 7 : kswz(r); };
  // (fixed bound: a bound that depends on GBK drops the host-side launch stub)
  unsigned va[8], vb[8];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int P = (i * NW + wave) * 64 + lane, r = P / CPR;
    const int kc = 8 * ((P % CPR) ^ swz(r));
    va[i] = row0 + r < M ? (unsigned)(((a_row(p, row0 + r) - ar0) * K + kc) * sizeof(TM))
                         : 0x80000000u;
    vb[i] = col0 + r < seg.width ? (unsigned)((r * K + kc) * sizeof(TB)) : 0x80000000u;
  }
  auto issue = [&](int kt, int stg) {
    const int ka = kt * GBK * (int)sizeof(TM), kb = kt * GBK * (int)sizeof(TB);
#pragma unroll
    for (int i = 0; i < NLD; ++i)  // token rows
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(lds + stg * STAGE + (i * NW + wave) * 512),
          16, va[i], ka, 0, 0);
#pragma unroll
    for (int i = 0; i < NLD; ++i)  // weight rows
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb,
          (__attribute__((address_space(3))) void*)(lds + stg * STAGE + TOK + (i * NW + wave) * 512),
          16, vb[i], kb, 0, 0);
  };
  auto frag_off = [&](int row, int chunk) { return row * GBK + 8 * (chunk ^ swz(row)); };

  // acc[i][j]: column block i (32 columns at CW wc + 32 i, i < NI) x token
  // block j (32 tokens at 128 wt + 32 j); fixed bounds, blocks i >= NI unused
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Software pipeline: the fragments of the next k-step are read from LDS
  // while the MFMAs of the current one run.  k-tile kt+1 is waited for and
  // published by the barrier between the two k-steps of tile kt (its second
  // k-step's fragments are already in registers by then), and the loads of
  // tile kt+3 go into the stage tile kt has just released.
  auto read_frags = [&](int stg, int ks, TMx8 (&a)[4], TMx8 (&b)[4]) {
    const TM* sa = lds + stg * STAGE;
    const TB* sb = (const TB*)(lds + stg * STAGE + TOK);
    const int ch = 2 * ks + lg;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const TBx8 w = *(const TBx8*)(sb + frag_off(CW * wc + 32 * i + lr, ch));
      if constexpr (__is_same(TM, TB))
        a[i] = w;
      else
        a[i] = __builtin_bit_cast(TMx8, bf16x8_to_f16x8(__builtin_bit_cast(u32x4, w)));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *(const TMx8*)(sa + frag_off(128 * wt + 32 * j + lr, ch));
  };
  auto mfmas = [&](const TMx8 (&a)[4], const TMx8 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  };
  // RoPE angles of the epilogue, fetched now so their latency hides under the
  // main loop (the loads are older than every tile load, so the loop's vmcnt
  // waits cover them)
  // (eight waves: no room for them in 256 registers)
  RopePre rp[2];
  const bool pre = NW == 4 && seg.kind == kHead && seg.rope;
  if (pre) {
    rope_prefetch<D>(p, row0, 0, rp[0]);
    rope_prefetch<D>(p, row0, 1, rp[1]);
  }
  // Each issue() is LPT loads per lane.  Wait until at most `n` later k-tiles
  // are still in flight (vmcnt(LPT n); NST - 2 >= n, so at most 16).
  // s_waitcnt vmcnt(N) with lgkmcnt and expcnt left alone: N's low 4 bits in
  // [3:0], its high 2 bits in [15:14]
  constexpr int W1 = (((1 * LPT) >> 4) << 14) | 0x0F70 | ((1 * LPT) & 15);
  constexpr int W2 = (((2 * LPT) >> 4) << 14) | 0x0F70 | ((2 * LPT) & 15);
  static_assert(2 * LPT < 64, "vmcnt holds 6 bits");
  auto wait_tiles = [](int n) {
    if (n >= 2)
      __builtin_amdgcn_s_waitcnt(W2);
    else if (n == 1)
      __builtin_amdgcn_s_waitcnt(W1);
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };
  const int nk = (K + GBK - 1) / GBK;
  for (int t = 0; t < NST - 1 && t < nk; ++t) issue(t, t);
  wait_tiles(min(nk - 1, NST - 2));  // tile 0 landed
  lds_barrier();
  if (NST - 1 < nk) issue(NST - 1, NST - 1);
  TMx8 fa[2][4], fb[2][4];
  read_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;  // KS is even: the parity carries over
      if (ks + 1 < KS) {
        read_frags(kt % NST, ks + 1, fa[nxt], fb[nxt]);
      } else if (kt + 1 < nk) {
        // tile kt+1 is complete for this lane once only tiles kt+2 .. kt+NST-1 remain
        wait_tiles(min(nk - 2 - kt, NST - 2));
        lds_barrier();  // tile kt+1 visible; every read of tile kt done
        if (kt + NST < nk) issue(kt + NST, (kt + NST) % NST);
        read_frags((kt + 1) % NST, 0, fa[nxt], fb[nxt]);
      }
      mfmas(fa[cur], fb[cur]);
    }
  }

  // Epilogue in two passes of 128 tokens (pass hf: token blocks 2hf, 2hf+1 of
  // both token halves, tile row 64 wt + 32 jj + lr), each written out as two
  // 128-column halves by the stores of the 256 x 128 kernel.  Register r of
  // acc[i][j] is tile column 128 wc + 32 i + 8 (r/4) + 4 lg + r%4.
  float* tile = (float*)smem;
  // hf is a compile-time constant, so acc is only ever indexed statically
  auto pass = [&](auto HF) {
    constexpr int hf = decltype(HF)::value;
    // LDS free (main loop, or the previous pass's stores).  LDS order only: a
    // __syncthreads() would also wait for this wave's global stores.
    lds_barrier();
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * hf + jj;
      const int trow = 64 * wt + 32 * jj + lr;
      if (seg.kind == kHeadT) {  // tile [column][token]
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = CW * wc + 32 * i + 8 * (r >> 2) + 4 * lg + (r & 3);
            tile[c * CP_ + trow] = acc[i][j][r];
          }
      } else {  // tile [token][column], float4 runs
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int c = CW * wc + 32 * i + 8 * a + 4 * lg;
            *(float4*)(tile + trow * RP_ + c) =
                make_float4(acc[i][j][4 * a], acc[i][j][4 * a + 1], acc[i][j][4 * a + 2],
                            acc[i][j][4 * a + 3]);
          }
      }
    }
    lds_barrier();  // the tile is in LDS
    // The stores are laid out for 256 threads and 128 columns: with 8 waves
    // each half of the workgroup writes one 128-column half of the tile.
    auto store_half = [&](int chh, int t) {
      if (seg.kind == kHeadT)
        store_cols<TO, D, CP_>(tile + 128 * chh * CP_, row0, hf, col0 + 128 * chh, seg, p, t);
      else if (seg.kind == kHead && seg.rope)
        store_rows_rope<TO, D, false, RP_>(tile + 128 * chh, row0, hf, col0 + 128 * chh, seg, p,
                                           pre ? &rp[hf] : nullptr, t);
      else
        store_rows_plain<TO, D, false, RP_>(tile + 128 * chh, row0, hf, col0 + 128 * chh, seg, p,
                                            t);
    };
    if constexpr (NW == 8) {
      store_half(wave >> 2, tid & 255);
    } else {
      store_half(0, tid);
      store_half(1, tid);
    }
  };
  pass(std::integral_constant<int, 0>{});
  pass(std::integral_constant<int, 1>{});
}

// --------------------------------------------------------------------------
// fp32 VALU GEMM (fp32 mode and the weight fold).  B(k, n) = Bp[k*sbk + n*sbn].
constexpr int SM = 64, SK = 16;

template <typename InT, typename OutT, int D>
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
      sAs[kk][r] = (gr < M && gk < K) ? to_f32(A[(size_t)a_row(p, gr) * K + gk]) : 0.f;
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
  epilogue_store<OutT, D, SM>(tile, row0, col0, seg, p);
}

SegTiles seg_tiles(const GemmProblem& p, int tn = BN) {
  SegTiles st{};
  int t = 0;
  for (int s = 0; s < p.nseg; ++s) {
    st.tile0[s] = t;
    t += (p.seg[s].width + tn - 1) / tn;
  }
  for (int s = p.nseg; s < 5; ++s) st.tile0[s] = t;
  return st;
}

}  // namespace

hipError_t launch_project_gemm(const GemmProblem& p, dar_dtype dt, hipStream_t s) {
  // the MFMA kernels stage whole k-tiles of 32 (d % 64 == 0, d_down % 32 == 0)
  if (dt == DAR_BF16 && p.K % 32 != 0) return hipErrorInvalidValue;
  // ragged rows: bf16 MFMA kernels, positions from the sequence starts only
  if (p.cu != nullptr && (dt != DAR_BF16 || p.row_pos != nullptr || p.n_cu < 1))
    return hipErrorInvalidValue;
  // sequences spread in A: whole sequences of n_seq rows, every A row under
  // 2 GiB of the start (the buffer resources' 32-bit offsets)
  if (p.a_ld_seq > 0) {
    const long last = (long)((p.M - 1) / p.n_seq) * p.a_ld_seq + (p.M - 1) % p.n_seq;
    if (p.a_ld_seq < p.n_seq || p.cu != nullptr || p.row_pos != nullptr ||
        (last + 1) * p.K * 2 > 0x7ffffff0L)
      return hipErrorInvalidValue;
  }
  const SegTiles st = seg_tiles(p);
  const int nC = st.tile0[p.nseg];
  if (dt == DAR_BF16 && p.row_pos == nullptr && p.b_type == kBF16) {
    // wide tiles once there are enough of them to fill every CU several times
    const SegTiles sw = seg_tiles(p, WBN);
    const int nCw = sw.tile0[p.nseg], nMw = (p.M + 255) / 256;
    // (bf16 activations: the first GEMM, long contractions; fp16: the global
    // GEMM of h^D, whose K = d_down is shorter but whose epilogue is half its time)
    if ((long)nCw * nMw >= kWideMinTiles && p.K % 64 == 0 &&
        ((p.K >= kWideMinK && p.a_type == kBF16) || (p.K >= 512 && p.a_type == kF16))) {
      size_t wbytes = 0;
      for (int i = 0; i < p.nseg; ++i) wbytes += (size_t)p.seg[i].width * p.K * 2;
      // a band's weights about fill one XCD's L2 (4 MB)
      const size_t tile_w = (size_t)WBN * p.K * 2;
      int band = (int)((size_t)kWideBandBytes / tile_w);
      band = band < 1 ? 1 : (band > nCw ? nCw : band);
      if (wbytes <= (size_t)(2 << 20)) band = nCw;
      const int total = nCw * nMw, per_xcd = (total + kNumXcd - 1) / kNumXcd;
      const dim3 grid(per_xcd * kNumXcd);
#define DAR_W(TA, TO, D)                                                                    \
  hipLaunchKernelGGL((project_gemm_wide<TA, bf16, TO, D, 64, 8>), grid, dim3(512), 0, s, p, sw, \
                     nMw, nCw, band, per_xcd)
      if (p.a_type == kBF16 && p.out_type == kF16) {
        if (p.d_k == 64) DAR_W(bf16, f16, 64); else DAR_W(bf16, f16, 128);
        return hipGetLastError();
      }
      if (p.a_type == kF16 && p.out_type == kF16) {
        if (p.d_k == 64) DAR_W(f16, f16, 64); else DAR_W(f16, f16, 128);
        return hipGetLastError();
      }
#undef DAR_W
    }
  }
  if (dt == DAR_BF16) {
    const int nM = (p.M + 2 * BM - 1) / (2 * BM);  // 256-token workgroup tiles
    const int nCp = (nC + kNumXcd - 1) / kNumXcd * kNumXcd;
    const int nMp = (nM + kNumXcd - 1) / kNumXcd * kNumXcd;
    // weights of every segment, in bytes: small enough for one XCD's L2 (4 MB)?
    size_t wbytes = 0;
    for (int i = 0; i < p.nseg; ++i) wbytes += (size_t)p.seg[i].width * p.K * 2;
    const int order = wbytes <= (size_t)(2 << 20) ? 1 : 0;
    const dim3 grid(order == 1 ? nMp * nC : nM * nCp);
#define DAR_G(TA, TO, D, RP)                                                         \
  hipLaunchKernelGGL((project_gemm_mfma<TA, bf16, TO, D, RP>), grid, dim3(256), 0, s, p, st, \
                     nM, nC, nCp, order)
    if (p.b_type != kBF16) return hipErrorInvalidValue;
    if (p.row_pos != nullptr) {  // ragged append: bf16 in and out only
      if (p.a_type != kBF16 || p.out_type != kBF16 || p.n_seq != 1) return hipErrorInvalidValue;
      if (p.d_k == 64) DAR_G(bf16, bf16, 64, true); else DAR_G(bf16, bf16, 128, true);
    } else if (p.a_type == kBF16 && p.out_type == kF16) {
      if (p.d_k == 64) DAR_G(bf16, f16, 64, false); else DAR_G(bf16, f16, 128, false);
    } else if (p.a_type == kF16 && p.out_type == kF16) {
      if (p.d_k == 64) DAR_G(f16, f16, 64, false); else DAR_G(f16, f16, 128, false);
    } else if (p.a_type == kBF16 && p.out_type == kBF16) {
      if (p.d_k == 64) DAR_G(bf16, bf16, 64, false); else DAR_G(bf16, bf16, 128, false);
    } else {
      return hipErrorInvalidValue;
    }
#undef DAR_G
  } else {
    const int nM = (p.M + SM - 1) / SM;
    if (p.d_k == 64)
      hipLaunchKernelGGL((gemm_simt<float, float, 64>), dim3(nC, nM), dim3(256), 0, s, p, st, 1L,
                         (long)p.K);
    else
      hipLaunchKernelGGL((gemm_simt<float, float, 128>), dim3(nC, nM), dim3(256), 0, s, p, st,
                         1L, (long)p.K);
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
  p.d_k = 64;  // unused by the row-major epilogue
  const SegTiles st = seg_tiles(p);
  const int nC = st.tile0[1], nM = (hd + SM - 1) / SM;
  if (dt == DAR_BF16)
    hipLaunchKernelGGL((gemm_simt<bf16, bf16, 64>), dim3(nC, nM), dim3(256), 0, s, p, st,
                       (long)d_down, 1L);
  else
    hipLaunchKernelGGL((gemm_simt<float, float, 64>), dim3(nC, nM), dim3(256), 0, s, p, st,
                       (long)d_down, 1L);
  return hipGetLastError();
}

}  // namespace dar
