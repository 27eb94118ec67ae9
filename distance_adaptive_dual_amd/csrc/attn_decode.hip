// Decode over the mixed cache.
//
// "Dual Dimensionality for Local and Global Attention": at inference a past
// token reaches a query through one source only, fixed by its distance (the
// remark after Eq. (5)), so the cache keeps full keys/values only for the w most recent positions and
// the d_down-wide latent h^D_j (Eq. 1) for every older position j.  For the
// query at position p:
//   j >  p - w : k_j, v_j read from the window ring (slot j mod w)
//   j <= p - w : k_j = RoPE_j(h^D_j W_upK), v_j = h^D_j W_upV   (Eqs. 2-3,
//                W_upK = W_up W_K and W_upV = W_up W_V folded once)
// and o = softmax(q K^T / sqrt(d_k)) V (Eq. 4).
//
// Keys of distant tokens must be rebuilt: RoPE at position j sits between
// W_upK and q, so W_upK cannot be absorbed into the query.  Values can: no
// rotation acts on them, so sum_j p_j h^D_j W_upV = (sum_j p_j h^D_j) W_upV
// and the latent kernel accumulates sum_j p_j h^D_j in d_down-space only.
//
// Two launches:
//  latent  -- one workgroup per (batch, head group, context chunk), 8 waves.
//             Each wave keeps 64 rows of W_upK^T in registers: 32 rotary
//             frequencies t of one head and their rotate-half partners
//             t + d_k/2, so a rebuilt key's two rotated components meet in one
//             lane.  32-token latent blocks stream through LDS (double
//             buffered); K'^T = W^T L^T on 32x32x16 MFMAs; RoPE + q.k per lane;
//             an online softmax per head; sum_j p_j h^D_j on 16x16x32 MFMAs.
//             Writes (max, sum, latent accumulator) per chunk.
//  window  -- extra workgroups of the same launch, one per (batch, head):
//             the w full keys/values.
//  combine -- log-sum-exp merge of all partials, then one lift by W_upV.
// Scores are kept in base 2 (log2(e)/sqrt(d_k) folded into q).
#include <math.h>

#include "dar_common.hpp"

namespace dar {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int TB = 32;        // tokens per latent block
constexpr int NWAVE = 8;      // waves per latent workgroup
constexpr int TARGET_WG = 1024;

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct DecodeGeom {
  int n_glob;      // latent positions 0 .. n_glob-1
  int n_chunks;    // context chunks per (batch, head group)
  int chunk_len;   // tokens per chunk (multiple of TB)
  int heads_per_wg;
  int n_hg;        // head groups
  int pairs;       // B * n_chunks, padded to a multiple of kNumXcd
  int n_win_pad;   // window workgroups (B * H), padded to a multiple of kNumXcd
  size_t part_lat_floats;  // per (b, head, chunk): 2 + d_down
};

DecodeGeom geom(const DecodeProblem& p) {
  DecodeGeom g{};
  const long pp = (long)p.ctx - 1;
  g.n_glob = (int)(pp - p.w + 1 > 0 ? pp - p.w + 1 : 0);
  g.heads_per_wg = NWAVE * 64 / p.d_k / (p.d_down > 256 ? 2 : 1);
  g.n_hg = (p.H + g.heads_per_wg - 1) / g.heads_per_wg;
  const int blocks = (g.n_glob + TB - 1) / TB;
  int want = TARGET_WG / (p.B * g.n_hg);
  if (want < 1) want = 1;
  if (want > blocks) want = blocks > 0 ? blocks : 1;
  const int bpc = (blocks + want - 1) / want > 0 ? (blocks + want - 1) / want : 1;
  g.chunk_len = bpc * TB;
  g.n_chunks = g.n_glob > 0 ? (g.n_glob + g.chunk_len - 1) / g.chunk_len : 1;
  g.pairs = (p.B * g.n_chunks + kNumXcd - 1) / kNumXcd * kNumXcd;
  g.part_lat_floats = 2 + (size_t)p.d_down;
  g.n_win_pad = (p.B * p.H + kNumXcd - 1) / kNumXcd * kNumXcd;
  return g;
}

// Context length of sequence b (ragged batches read it from the device,
// clamped to [1, ctx]).
__device__ __forceinline__ int seq_ctx(const DecodeProblem& p, int b) {
  if (p.ctx_lens == nullptr) return p.ctx;
  const int c = p.ctx_lens[b];
  return c < 1 ? 1 : (c > p.ctx ? p.ctx : c);
}

// --------------------------------------------------------------------------
constexpr float kTau = 8.f;        // move the reference max only past 2^8 growth
constexpr float kNegBig = -1e30f;

template <int D, int KS>
struct LatentSmem {
  static constexpr int DD = KS * 16;   // d_down
  static constexpr int NBUF = KS <= 16 ? 4 : 3;  // latent ring depth
  static constexpr int CP = D / 2 + 2; // float2 per cos/sin row (16 B pad)
  // latent blocks [token][d_down] with rows LP = d_down + 8 apart: the
  // 16-byte pad puts consecutive rows read at one column in different bank
  // groups
  static constexpr int LP = DD + 8;
  bf16 lat[NBUF][TB * LP];
  float2 cs[2][TB * CP];               // (cos, sin)(j theta_t) of a block, [token][t]
  float sc[2][NWAVE][TB];              // per-wave partial scores
  bf16 pm[2][16][TB + 8];              // probabilities, rows = heads of the group
  float alpha[2][16];                  // per-head rescale of this block
};

// Per (batch, head group, context chunk); 8 waves of 64 rows each.
//
// A wave keeps, for one head h and 32 rotary frequencies t, the rows W_t and
// W_{t+d_k/2} of W_upK^T in registers and folds the (pre-rotated) query into
// them once:  alpha_t = q_t W_t + q_{t+h} W_{t+h},  beta_t = q_{t+h} W_t - q_t W_{t+h}.
// For a latent h^D_j the rotated key k_j = RoPE_j(h^D_j W_upK) then satisfies
//   q . k_j = sum_t cos(j theta_t) (h^D_j . alpha_t) + sin(j theta_t) (h^D_j . beta_t)
// (expand the rotate-half rotation), so one 32x32x16 MFMA chain over d_down
// gives h^D . alpha and h^D . beta for 32 tokens and the score needs two FMAs
// per frequency.  cos/sin(j theta_t) advance by one complex multiply per
// 32-token block (the fine table's row 32), starting from the fp64 tables.
// --------------------------------------------------------------------------
// Window part: the min(w, ctx) ring slots that hold positions p-w+1 .. p (the
// set of valid slots is always 0 .. nw-1; its order does not matter to a
// softmax).  Run by extra workgroups of the latent launch, one per (batch,
// head): 64-key chunks staged in LDS with 16-byte loads, eight lanes per key
// for the scores, online softmax.
template <int D>
struct WindowSmem {
  static constexpr int CK = 64, KP = D + 8;
  bf16 ks[CK * KP];
  bf16 vs[CK * KP];
  float sc[CK];
  float accs[512 / D][D];
};

template <int D>
__device__ void window_part(const DecodeProblem& p, float* part_win, int bh, WindowSmem<D>& sm) {
  constexpr int CK = WindowSmem<D>::CK, KP = WindowSmem<D>::KP, NT = 512;
  const int tid = threadIdx.x;
  const int ctx_b = seq_ctx(p, bh / p.H);
  const int nw = ctx_b < p.w ? ctx_b : p.w;
  const float scl = kLog2e / sqrtf((float)D);
  const bf16* qp = (const bf16*)p.q + (size_t)bh * D;
  const bf16* Kw = (const bf16*)p.K_win + (size_t)bh * p.w * D;
  const bf16* Vw = (const bf16*)p.V_win + (size_t)bh * p.w * D;
  // score lanes: key kq = tid / 8, dims pt + 8 e
  const int kq = tid >> 3, pt = tid & 7;
  float qv[D / 8];
#pragma unroll
  for (int e = 0; e < D / 8; ++e) qv[e] = (float)qp[pt + 8 * e] * scl;
  // value lanes: dim vd, keys vk, vk + NT/D, ...
  constexpr int KPB = NT / D;
  const int vd = tid % D, vk = tid / D;
  float m_run = kNegBig, l_run = 0.f, acc = 0.f;
  for (int c0 = 0; c0 < nw; c0 += CK) {
    const int nk = min(CK, nw - c0);
    __syncthreads();
    for (int c = tid; c < CK * D / 8; c += NT) {
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (r < nk) {
        kv = *(const u32x4*)(Kw + (size_t)(c0 + r) * D + col);
        vv = *(const u32x4*)(Vw + (size_t)(c0 + r) * D + col);
      }
      *(u32x4*)(sm.ks + r * KP + col) = kv;
      *(u32x4*)(sm.vs + r * KP + col) = vv;
    }
    __syncthreads();
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < D / 8; ++e) dot = fmaf(qv[e], (float)sm.ks[kq * KP + pt + 8 * e], dot);
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    dot += __shfl_xor(dot, 4);
    if (pt == 0) sm.sc[kq] = kq < nk ? dot : -INFINITY;
    __syncthreads();
    float mt = -INFINITY;
    for (int i = 0; i < CK; ++i) mt = fmaxf(mt, sm.sc[i]);
    const float m_new = fmaxf(m_run, mt);
    const float al = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float ls = 0.f;
    acc *= al;
    for (int i = 0; i < CK; ++i) {
      const float e = __builtin_amdgcn_exp2f(sm.sc[i] - m_new);
      ls += e;
      if ((i % KPB) == vk) acc = fmaf(e, (float)sm.vs[i * KP + vd], acc);
    }
    l_run = l_run * al + ls;
  }
  sm.accs[vk][vd] = acc;
  __syncthreads();
  float* dst = part_win + (size_t)bh * (2 + D);
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < KPB; ++i) a += sm.accs[i][tid];
    dst[2 + tid] = a;
  }
  if (tid == 0) {
    dst[0] = nw > 0 ? m_run : -INFINITY;
    dst[1] = l_run;
  }
}

template <int D, int KS>
__global__ __launch_bounds__(512, 1) void decode_latent(DecodeProblem p, DecodeGeom g,
                                                    float* part_win) {
  using S = LatentSmem<D, KS>;
  // NS: slices of d_down per frequency block (a wave holds the folded rows of
  // 32 frequencies over d_down / NS latent dims: at most 128 VGPRs).
  constexpr int DD = S::DD, LP = S::LP, NBUF = S::NBUF, CP = S::CP, WPH = D / 64, HALF = D / 2;
  constexpr int NS = KS > 16 ? 2 : 1, KSW = KS / NS, WPHS = WPH * NS, HPW = NWAVE / WPHS;
  union Smem {
    S lat;
    WindowSmem<D> win;
  };
  __shared__ Smem smu;
  S& sm = smu.lat;

  // The first n_win_pad workgroups do the window part (one per (batch,
  // head)); they start first and overlap the latent stream.
  if ((int)blockIdx.x < g.n_win_pad) {
    if ((int)blockIdx.x < p.B * p.H) window_part<D>(p, part_win, blockIdx.x, smu.win);
    return;
  }
  // XCD-aware order: the head groups of one (batch, chunk) run on one XCD so
  // its latent block is fetched from HBM once and served to the rest by L2.
  const int bid = blockIdx.x - g.n_win_pad;
  const int x = bid % kNumXcd, k = bid / kNumXcd;
  const int pair = x + kNumXcd * (k / g.n_hg), hg = k % g.n_hg;
  if (pair >= p.B * g.n_chunks) return;
  const int b = pair / g.n_chunks, chunk = pair % g.n_chunks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lg = lane >> 5;
  // wave -> head hl of the group, frequency block tb, d_down slice sl
  const int hl = wave / WPHS, wih = wave % WPHS, tb = wih / NS, sl = wih % NS;
  const int head = hg * HPW + hl;
  const bool head_ok = head < p.H;

  const int j_begin = chunk * g.chunk_len;
  const int n_glob_b = p.ctx_lens ? max(seq_ctx(p, b) - p.w, 0) : g.n_glob;
  const int j_end = min(n_glob_b, j_begin + g.chunk_len);
  const int nblk = j_end > j_begin ? (j_end - j_begin + TB - 1) / TB : 0;

  // Query-folded weight rows (MFMA A operand): row t = 32 tb + lr of this
  // lane and its partner t + D/2; scores come out in base-2 logits.
  bf16x8 gf[2][KSW];
  {
    const bf16* Wk = (const bf16*)p.W_upK;
    const int hh = head_ok ? head : 0;
    const int t = 32 * tb + lr;
    const bf16* qp = (const bf16*)p.q + ((size_t)b * p.H + hh) * D;
    const float scl = kLog2e / sqrtf((float)D);
    const float qa = (float)qp[t] * scl, qb = (float)qp[t + HALF] * scl;
    const bf16* r0 = Wk + (size_t)(hh * D + t) * DD + 16 * KSW * sl + 8 * lg;
    const bf16* r1 = r0 + (size_t)HALF * DD;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const bf16x8 w0 = *(const bf16x8*)(r0 + 16 * ks), w1 = *(const bf16x8*)(r1 + 16 * ks);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = (float)w0[e], c = (float)w1[e];
        gf[0][ks][e] = (bf16)(a * qa + c * qb);
        gf[1][ks][e] = (bf16)(a * qb - c * qa);
      }
    }
  }
  // cos/sin(j theta_t) of the current block go through LDS, shared by every
  // wave: thread tid carries frequency t = tid % (D/2) for NE tokens of the
  // block and advances them by one complex multiply with (cos, sin)(32 theta_t)
  // per block, starting from the fp64 tables at the chunk's first position.
  constexpr int NE = TB * HALF / 512, TSTEP = 512 / HALF;
  const int ct = tid % HALF, ctok = tid / HALF;
  const float2 cstep = p.rope.lo[32 * HALF + ct];
  float2 cst[NE];
#pragma unroll
  for (int i = 0; i < NE; ++i) cst[i] = rope_cs(p.rope, j_begin + ctok + TSTEP * i, ct);
  // table of the next block into cs[buf]; the state moves one block on
  auto put_cs = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      sm.cs[buf][(ctok + TSTEP * i) * CP + ct] = cst[i];
      const float c = cst[i].x * cstep.x - cst[i].y * cstep.y;
      cst[i].y = cst[i].x * cstep.y + cst[i].y * cstep.x;
      cst[i].x = c;
    }
  };

  // Latent blocks go from HBM straight into LDS (buffer loads with an LDS
  // destination, no registers): one load per token row, its 2 KS lanes writing
  // 16 bytes each from the row's start (the other lanes idle), wave w loading
  // rows w, w + 8, ...  The buffer covers this chunk's rows only, so rows past
  // j_end read as zeros.
  const __amdgpu_buffer_rsrc_t lrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const bf16*)p.h_D + ((size_t)b * p.cap + j_begin) * DD), (short)0,
      (int)((size_t)(j_end > j_begin ? j_end - j_begin : 0) * DD * sizeof(bf16)), 0x00020000);
  constexpr int CPR = 2 * KS;  // 16-byte chunks per latent row
  auto issue_blk = [&](int blk) {
    bf16* dst = sm.lat[blk % NBUF];
#pragma unroll
    for (int i = 0; i < TB / NWAVE; ++i) {
      const int row = wave + NWAVE * i;
      if (CPR == 64 || lane < CPR) {
        const unsigned off = (unsigned)(((blk * TB + row) * DD + 8 * lane) * sizeof(bf16));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            lrs, (__attribute__((address_space(3))) void*)(dst + row * LP), 16, off, 0, 0, 0);
      }
    }
  };

  // softmax state, kept by the first wave of each head (lanes 0..31 own tokens)
  float m_ref = kNegBig, l_lane = 0.f;
  constexpr int NB = DD / 16;
  constexpr int NB_PER_WAVE = (NB + NWAVE - 1) / NWAVE;
  f32x4 acc[NB_PER_WAVE];
#pragma unroll
  for (int i = 0; i < NB_PER_WAVE; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // acc[head, dims] = alpha * acc + P L for block `blk` (16x16x32 MFMA, K = the
  // 32 tokens).  Contraction slot c of lane group kg is token 8*(c/2) + 2*kg +
  // c%2: both operands use that order, and the four groups then read latent
  // rows two apart, which fall in disjoint LDS banks.
  auto accumulate = [&](int blk) {
    const int pb = blk & 1;
    const bf16* L = sm.lat[blk % NBUF];
#pragma unroll
    for (int i = 0; i < NB_PER_WAVE; ++i) {
      const int nb = wave + NWAVE * i;
      if (nb < NB) {
        const int row = lane & 15, kg = lane >> 4;
        bf16x8 af;
        if (row < HPW) {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t two = *(const uint32_t*)(&sm.pm[pb][row][8 * m + 2 * kg]);
            af[2 * m] = __builtin_bit_cast(bf16, (uint16_t)(two & 0xffffu));
            af[2 * m + 1] = __builtin_bit_cast(bf16, (uint16_t)(two >> 16));
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) af[c] = (bf16)0.f;
        }
        bf16x8 bfr;
        const int n = nb * 16 + row;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          bfr[c] = L[(8 * (c >> 1) + 2 * kg + (c & 1)) * LP + n];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hrow = 4 * kg + r;
          acc[i][r] *= (hrow < HPW) ? sm.alpha[pb][hrow] : 1.f;
        }
        acc[i] = mfma16x16x32(af, bfr, acc[i]);
      }
    }
  };

  // Block k lives in lat[k % NBUF].  Its loads are issued after barrier k - 2
  // and waited for (each wave its own) just before barrier k - 1, so they
  // have a whole block's work to land in.  With a ring of four there is one
  // barrier per block: barrier k publishes the partial scores of block k, the
  // probabilities of block k - 1, the cos/sin table of block k + 1 and the
  // latents of block k + 1, and frees lat[(k + 2) % 4] (block k - 2, whose
  // value sum ran before barrier k).  With a ring of three (the widest
  // latents, for LDS room) a second barrier precedes the value sum of block k
  // itself, and lat[(k + 2) % 3] (block k - 1) is free after barrier k.
  if (nblk > 0) issue_blk(0);
  if (nblk > 1) issue_blk(1);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  put_cs(0);
  __syncthreads();

  // Scores of block blk into sc[blk % 2]; cos/sin table of block blk + 1.
  auto scores = [&](int blk) {
    const int pb = blk & 1;
    // h^D . [alpha | beta] for 32 tokens (lane column lr)
    const bf16* lrow = sm.lat[blk % NBUF] + lr * LP + 16 * KSW * sl + 8 * lg;
    // the cos/sin table of the 4 frequency groups: read before the MFMAs when
    // the registers allow it without lowering occupancy (d_down >= 256;
    // 0.575 -> 0.570 ms at ctx 32768), after them otherwise
    const float2* crow = &sm.cs[pb][lr * CP + 32 * tb + 4 * lg];
    f32x4 cx[4], cy[4];
    if constexpr (KS >= 16) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        cx[g] = *(const f32x4*)(crow + 8 * g);
        cy[g] = *(const f32x4*)(crow + 8 * g + 2);
      }
    }
    f32x16 kc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) kc[mb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const bf16x8 lf = *(const bf16x8*)(lrow + 16 * ks);
      kc[0] = mfma32x32x16(gf[0][ks], lf, kc[0]);
      kc[1] = mfma32x32x16(gf[1][ks], lf, kc[1]);
    }
    // output register r holds frequency t = 32 tb + 8 (r/4) + 4 lg + r%4 of
    // token j0 + lr: four consecutive frequencies per r/4, 32 bytes of the table
    float sp = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 x, y;
      if constexpr (KS >= 16) {
        x = cx[g];
        y = cy[g];
      } else {
        x = *(const f32x4*)(crow + 8 * g);
        y = *(const f32x4*)(crow + 8 * g + 2);
      }
      sp = fmaf(x[0], kc[0][4 * g], fmaf(x[1], kc[1][4 * g], sp));
      sp = fmaf(x[2], kc[0][4 * g + 1], fmaf(x[3], kc[1][4 * g + 1], sp));
      sp = fmaf(y[0], kc[0][4 * g + 2], fmaf(y[1], kc[1][4 * g + 2], sp));
      sp = fmaf(y[2], kc[0][4 * g + 3], fmaf(y[3], kc[1][4 * g + 3], sp));
    }
    sp += __shfl_xor(sp, 32);
    if (lg == 0) sm.sc[pb][wave][lr] = sp;
    put_cs(pb ^ 1);
  };
  // Probabilities of block blk (sc[blk % 2] -> pm, alpha), kept by the first
  // wave of each head.
  auto softmax = [&](int blk) {
    const int pb = blk & 1;
    const int j0 = j_begin + blk * TB;
    if (wih == 0) {
      // score of token j0 + lr for head hl (both lane halves hold it): the
      // partial sums of the head's WPHS waves
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < WPHS; ++i) s += sm.sc[pb][wave + i][lr];
      const bool ok = head_ok && (j0 + lr < j_end);
      s = ok ? s : -INFINITY;
      float al = 1.f;
      if (__builtin_amdgcn_ballot_w64(s > m_ref + kTau) != 0) {
        float mt = s;
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
        const float m_new = fmaxf(m_ref, mt);
        al = __builtin_amdgcn_exp2f(m_ref - m_new);
        m_ref = m_new;
        l_lane *= al;
      }
      const float e = __builtin_amdgcn_exp2f(s - m_ref);
      const bf16 eb = (bf16)e;
      if (lg == 0) {
        l_lane += (float)eb;  // the sum of exactly the probabilities used below
        sm.pm[pb][hl][lr] = eb;
      }
      if (lane == 0) sm.alpha[pb][hl] = al;
    }
  };

  if constexpr (NBUF == 4) {
    // Iteration blk runs between barriers blk - 1 and blk: the loads of block
    // blk + 1, the scores of block blk, the probabilities of block blk - 1 and
    // the value sum of block blk - 2, in either order (each reads only what
    // barrier blk - 1 published).  The waves of the upper half take the
    // probabilities and value sum first, so the two waves that share a SIMD
    // are out of phase: one issues MFMAs while the other runs VALU work.
    const bool post_first = wave >= NWAVE / 2;
    for (int blk = 0; blk < nblk; ++blk) {
      if (blk > 0 && blk + 1 < nblk) issue_blk(blk + 1);
      if (post_first && blk > 0) {
        softmax(blk - 1);
        if (blk > 1) accumulate(blk - 2);
      }
      scores(blk);
      if (!post_first && blk > 0) {
        softmax(blk - 1);
        if (blk > 1) accumulate(blk - 2);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block blk + 1
      __syncthreads();
    }
    if (nblk > 0) {
      softmax(nblk - 1);
      if (nblk > 1) accumulate(nblk - 2);
      __syncthreads();  // probabilities of the last block
      accumulate(nblk - 1);
    }
  } else {
    for (int blk = 0; blk < nblk; ++blk) {
      scores(blk);
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of block blk + 1
      __syncthreads();
      if (blk + 2 < nblk) issue_blk(blk + 2);
      softmax(blk);
      __syncthreads();  // probabilities of block blk visible
      accumulate(blk);
    }
  }

  // partials: part[((b*H + head)*n_chunks + chunk)] = {m, l, acc[d_down]}
  float* part = (float*)p.ws;
  if (wih == 0) {
    float l = l_lane;
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) l += __shfl_xor(l, off);
    if (lane == 0 && head_ok) {
      float* dst = part + (((size_t)b * p.H + head) * g.n_chunks + chunk) * g.part_lat_floats;
      dst[0] = m_ref;
      dst[1] = l;
    }
  }
#pragma unroll
  for (int i = 0; i < NB_PER_WAVE; ++i) {
    const int nb = wave + NWAVE * i;
    if (nb < NB) {
      const int col = nb * 16 + (lane & 15), kg = lane >> 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hrow = 4 * kg + r, hh = hg * HPW + hrow;
        if (hrow < HPW && hh < p.H) {
          float* dst = part + (((size_t)b * p.H + hh) * g.n_chunks + chunk) * g.part_lat_floats;
          dst[2 + col] = acc[i][r];
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// Merge: o_h = (acc_lat W_upV_h + acc_win) / l with every partial rescaled to
// the common maximum.
template <int D>
__global__ __launch_bounds__(256) void decode_combine(DecodeProblem p, DecodeGeom g,
                                                      const float* part_lat,
                                                      const float* part_win, int n_win) {
  __shared__ float lat[1024];
  __shared__ float wsc[1024];
  __shared__ float wwf[64];
  __shared__ float wacc[D];
  __shared__ float red[2];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int DD = p.d_down, nc = g.n_chunks;
  const size_t PF = g.part_lat_floats;
  const float* pl = part_lat + (size_t)bh * nc * PF;
  // window partials (max, sum, acc[D]) of this (batch, head): n_win in a row
  const float* pw = part_win + (size_t)bh * n_win * (2 + D);
  // The loads that do not depend on the merge weights go out first, so their
  // latency overlaps the weights': the lift's W_upV row piece (TPR threads
  // per output row t, DD / TPR columns each, 16-byte chunks) and this
  // thread's latent column of the first CPF partials.
  constexpr int TPR = 256 / D, WPF = 16, CPF = 32, NWP = 4;
  const int h = bh % p.H;
  const bf16* Wv = (const bf16*)p.W_upV + (size_t)h * D * DD;
  const int t = tid / TPR, part = tid % TPR;
  const int per = DD / TPR;  // a multiple of 8 for every supported d_down
  const bf16* wr = Wv + (size_t)t * DD + part * per;
  bf16x8_t wv[WPF];
#pragma unroll
  for (int i = 0; i < WPF; ++i)
    if (8 * i < per) wv[i] = *(const bf16x8_t*)(wr + 8 * i);
  float pv[CPF];
#pragma unroll
  for (int c = 0; c < CPF; ++c) pv[c] = (tid < DD && c < nc) ? pl[c * PF + 2 + tid] : 0.f;
  // and this thread's column of the first NWP window partials
  float wp[NWP];
#pragma unroll
  for (int k = 0; k < NWP; ++k) wp[k] = (tid < D && k < n_win) ? pw[k * (2 + D) + 2 + tid] : 0.f;
  if (wave == 0) {
    // common maximum over the non-empty partials, their weights and the total
    float M = (lane < n_win && pw[lane * (2 + D) + 1] > 0.f) ? pw[lane * (2 + D)] : -INFINITY;
    for (int c = lane; c < nc; c += 64)
      if (pl[c * PF + 1] > 0.f) M = fmaxf(M, pl[c * PF]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    float L = 0.f;
    for (int c = lane; c < nc; c += 64) {
      const float* e = pl + c * PF;
      const float f = (e[1] > 0.f) ? exp2f(e[0] - M) : 0.f;
      wsc[c] = f;
      L += f * e[1];
    }
    if (lane < n_win) {
      const float* e = pw + lane * (2 + D);
      const float f = (e[1] > 0.f) ? exp2f(e[0] - M) : 0.f;
      wwf[lane] = f;
      L += f * e[1];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) L += __shfl_xor(L, off);
    if (lane == 0) red[1] = L;
  }
  __syncthreads();
  // the window's value sum in d_k space
  if (tid < D) {
    float a = 0.f;
#pragma unroll
    for (int k = 0; k < NWP; ++k)
      if (k < n_win) a = fmaf(wwf[k], wp[k], a);
    for (int k = NWP; k < n_win; ++k) a = fmaf(wwf[k], pw[k * (2 + D) + 2 + tid], a);
    wacc[tid] = a;
  }
  // latent sum: a thread per latent column (the first CPF partials from the
  // prefetched values)
  if (tid < DD) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CPF; ++c)
      if (c < nc) a[c & 3] = fmaf(wsc[c], pv[c], a[c & 3]);
    for (int c = CPF; c < nc; ++c) a[c & 3] = fmaf(wsc[c], pl[c * PF + 2 + tid], a[c & 3]);
    lat[tid] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  for (int kk = tid + 256; kk < DD; kk += 256) {
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nc; ++c) a[c & 3] = fmaf(wsc[c], pl[c * PF + 2 + kk], a[c & 3]);
    lat[kk] = (a[0] + a[1]) + (a[2] + a[3]);
  }
  __syncthreads();
  // lift by W_upV, partial sums of a row met by shuffles
  const float inv = 1.f / red[1];
  const float* lp = lat + part * per;
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < WPF; ++i)
    if (8 * i < per) {
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(lp[8 * i + e], (float)wv[i][e], a);
    }
  for (int kk = 8 * WPF; kk < per; kk += 8) {
    const bf16x8_t v = *(const bf16x8_t*)(wr + kk);
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaf(lp[kk + e], (float)v[e], a);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) a += __shfl_xor(a, off);
  if (part == 0) ((bf16*)p.o)[(size_t)bh * D + t] = (bf16)((a + wacc[t]) * inv);
}

template <int D, int KS>
hipError_t launch_latent(const DecodeProblem& p, const DecodeGeom& g, float* part_win,
                         hipStream_t s) {
  const int grid = g.n_win_pad + g.pairs * g.n_hg;
  hipLaunchKernelGGL((decode_latent<D, KS>), dim3(grid), dim3(512), 0, s, p, g, part_win);
  return hipGetLastError();
}

}  // namespace

size_t decode_workspace_bytes(const DecodeProblem& p) {
  const DecodeGeom g = geom(p);
  const size_t lat = sizeof(float) * (size_t)p.B * p.H * g.n_chunks * g.part_lat_floats;
  const size_t win = sizeof(float) * (size_t)p.B * p.H * (2 + p.d_k);
  return ((lat + 255) & ~(size_t)255) + ((win + 255) & ~(size_t)255);
}

hipError_t launch_attn_decode(const DecodeProblem& p, hipStream_t s) {
  const DecodeGeom g = geom(p);
  float* part_lat = (float*)p.ws;
  const size_t lat = sizeof(float) * (size_t)p.B * p.H * g.n_chunks * g.part_lat_floats;
  float* part_win = (float*)((char*)p.ws + ((lat + 255) & ~(size_t)255));
  hipError_t e = hipSuccess;
  const int KS = p.d_down / 16;
#define DAR_LAT(DV, KV) \
  if (p.d_k == DV && KS == KV) e = launch_latent<DV, KV>(p, g, part_win, s);
  DAR_LAT(64, 2)
  DAR_LAT(64, 4)
  DAR_LAT(64, 8)
  DAR_LAT(64, 16)
  DAR_LAT(64, 32)
  DAR_LAT(128, 2)
  DAR_LAT(128, 4)
  DAR_LAT(128, 8)
  DAR_LAT(128, 16)
  DAR_LAT(128, 32)
#undef DAR_LAT
  if (e != hipSuccess) return e;
  if (p.d_k == 64)
    hipLaunchKernelGGL(decode_combine<64>, dim3(p.B * p.H), dim3(256), 0, s, p, g, part_lat,
                       part_win, 1);
  else
    hipLaunchKernelGGL(decode_combine<128>, dim3(p.B * p.H), dim3(256), 0, s, p, g, part_lat,
                       part_win, 1);
  return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeProblem& p, int n_chunks, const float* part_lat,
                                 const float* part_win, int n_win, hipStream_t s) {
  DecodeGeom g{};
  g.n_chunks = n_chunks;
  g.part_lat_floats = 2 + (size_t)p.d_down;
  if (p.d_k == 64)
    hipLaunchKernelGGL(decode_combine<64>, dim3(p.B * p.H), dim3(256), 0, s, p, g, part_lat,
                       part_win, n_win);
  else
    hipLaunchKernelGGL(decode_combine<128>, dim3(p.B * p.H), dim3(256), 0, s, p, g, part_lat,
                       part_win, n_win);
  return hipGetLastError();
}

bool decode_supported(int d_k, int d_down) {
  const int KS = d_down / 16;
  return (d_k == 64 || d_k == 128) && d_down % 16 == 0 &&
         (KS == 2 || KS == 4 || KS == 8 || KS == 16 || KS == 32);
}

}  // namespace dar
