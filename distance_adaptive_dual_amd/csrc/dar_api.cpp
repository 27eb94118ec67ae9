// C ABI of the DAR attention library: argument validation, workspace sizing
// and launches on the caller's stream.  No allocation, no state, no host
// synchronisation.  The kernels live in rope.hip, gemm.hip, attn_prefill.hip,
// attn_decode.hip and cache.hip.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "dar_common.hpp"

using namespace dar;

namespace {

constexpr int kAbiVersion = 2;

size_t elem_size(dar_dtype dt) { return dt == DAR_BF16 ? 2 : 4; }
bool dtype_ok(dar_dtype dt) { return dt == DAR_BF16 || dt == DAR_FP32; }
bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

struct Span {
  const void* p;
  size_t bytes;
};

bool overlap(const Span& a, const Span& b) {
  if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// Every output must be disjoint from every input and every other output.
bool disjoint(const Span* outs, int nout, const Span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return false;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return false;
  }
  return true;
}

// Limits of the kernels (DAR_ERR_UNSUPPORTED beyond them).
bool head_supported(int d_k) { return d_k == 64 || d_k == 128; }

dar_status hip_status(hipError_t e) { return e == hipSuccess ? DAR_OK : DAR_ERR_HIP; }

}  // namespace

extern "C" {

int dar_abi_version(void) { return kAbiVersion; }

const char* dar_status_string(dar_status s) {
  switch (s) {
    case DAR_OK: return "DAR_OK";
    case DAR_ERR_INVALID_ARG: return "DAR_ERR_INVALID_ARG";
    case DAR_ERR_UNSUPPORTED: return "DAR_ERR_UNSUPPORTED";
    case DAR_ERR_WORKSPACE: return "DAR_ERR_WORKSPACE";
    case DAR_ERR_HIP: return "DAR_ERR_HIP";
  }
  return "DAR_ERR_UNKNOWN";
}

dar_status dar_fold(const void* W_up, const void* W_K, const void* W_V, int d, int d_down,
                    int heads, int d_k, dar_dtype dtype, void* W_upK, void* W_upV,
                    hipStream_t stream) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1)) return DAR_ERR_INVALID_ARG;
  if (!aligned16(W_up) || !aligned16(W_K) || !aligned16(W_V) || !aligned16(W_upK) ||
      !aligned16(W_upV))
    return DAR_ERR_INVALID_ARG;
  const int hd = heads * d_k;
  const size_t es = elem_size(dtype);
  const Span ins[3] = {{W_up, es * d_down * d}, {W_K, es * d * hd}, {W_V, es * d * hd}};
  const Span outs[2] = {{W_upK, es * d_down * hd}, {W_upV, es * d_down * hd}};
  if (!disjoint(outs, 2, ins, 3)) return DAR_ERR_INVALID_ARG;
  if (!head_supported(d_k) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;
  hipError_t e = launch_fold(W_up, W_K, W_upK, d, d_down, hd, dtype, stream);
  if (e == hipSuccess) e = launch_fold(W_up, W_V, W_upV, d, d_down, hd, dtype, stream);
  return hip_status(e);
}

// act: 0 for Eq. (1) as written, 1 for the sigmoid after the down-projection.
static dar_status project_impl(const void* h, const void* W_down, const void* W_up,
                               const void* W_Q, const void* W_K, const void* W_V,
                               const void* W_upK, const void* W_upV, int B, int N, int d,
                               int d_down, int heads, int d_k, int pos0, float rope_base,
                               dar_dtype dtype, void* Q, void* K_loc, void* V_loc, void* h_D,
                               void* K_glob, void* V_glob, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream, int act,
                               const int* cu = nullptr, int n_cu = 0, int max_len = 0) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1) || pos0 < 0)
    return DAR_ERR_INVALID_ARG;
  if (!(rope_base > 1.0f)) return DAR_ERR_INVALID_ARG;
  if ((long)pos0 + N - 1 > 0x7fffffffL) return DAR_ERR_INVALID_ARG;
  const bool have_fold = (W_upK != nullptr) || (W_upV != nullptr);
  if (have_fold && (!aligned16(W_upK) || !aligned16(W_upV))) return DAR_ERR_INVALID_ARG;
  if (!have_fold && !aligned16(W_up)) return DAR_ERR_INVALID_ARG;
  const void* need[] = {h, W_down, W_Q, W_K, W_V, Q, K_loc, V_loc, h_D, K_glob, V_glob};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const int hd = heads * d_k;
  const size_t es = elem_size(dtype);
  const size_t M = (size_t)B * N;
  const Span ins[8] = {{h, es * M * d},           {W_down, es * d * d_down},
                       {W_Q, es * d * hd},        {W_K, es * d * hd},
                       {W_V, es * d * hd},        {have_fold ? nullptr : W_up, es * d_down * d},
                       {W_upK, es * d_down * hd}, {W_upV, es * d_down * hd}};
  const Span outs[6] = {{Q, es * M * hd},    {K_loc, es * M * hd}, {V_loc, es * M * hd},
                        {h_D, es * M * d_down}, {K_glob, es * M * hd}, {V_glob, es * M * hd}};
  if (!disjoint(outs, 6, ins, 8)) return DAR_ERR_INVALID_ARG;
  if (!head_supported(d_k) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;

  // ragged rows: positions 0 .. max_len - 1 within each sequence
  const long max_pos = cu != nullptr ? (long)max_len - 1 : (long)pos0 + N - 1;
  const size_t rope_bytes = rope_table_bytes(d_k, max_pos);
  const size_t fold_bytes = have_fold ? 0 : 2 * round256(es * d_down * hd);
  const size_t need_bytes = rope_bytes + fold_bytes;
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& s : ins)
      if (overlap(ws, s)) return DAR_ERR_INVALID_ARG;
    for (const Span& s : outs)
      if (overlap(ws, s)) return DAR_ERR_INVALID_ARG;
  }

  char* wsp = (char*)workspace;
  float2* lo = (float2*)wsp;
  float2* hi = lo + 64 * (d_k / 2);
  hipError_t e = launch_rope_tables(lo, hi, d_k, max_pos, rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  const void* fK = W_upK;
  const void* fV = W_upV;
  if (!have_fold) {
    void* k_out = wsp + rope_bytes;
    void* v_out = wsp + rope_bytes + round256(es * d_down * hd);
    e = launch_fold(W_up, W_K, k_out, d, d_down, hd, dtype, stream);
    if (e == hipSuccess) e = launch_fold(W_up, W_V, v_out, d, d_down, hd, dtype, stream);
    if (e != hipSuccess) return DAR_ERR_HIP;
    fK = k_out;
    fV = v_out;
  }
  const RopeTab rope{lo, hi, d_k / 2};

  GemmProblem g1{};
  const bool bf = dtype == DAR_BF16;
  g1.A = h;
  g1.M = (int)M;
  g1.K = d;
  g1.a_type = bf ? kBF16 : kF32;
  g1.b_type = bf ? kBF16 : kF32;
  g1.out_type = bf ? kF16 : kF32;
  g1.nseg = 4;
  g1.seg[0] = GemmSeg{W_Q, Q, hd, kHead, 1};
  g1.seg[1] = GemmSeg{W_K, K_loc, hd, kHead, 1};
  g1.seg[2] = GemmSeg{W_V, V_loc, hd, kHeadT, 0};
  g1.seg[3] = GemmSeg{W_down, h_D, d_down, kRowMajor, 0};
  g1.seg[3].act = act;
  g1.n_seq = N;
  g1.heads = heads;
  g1.d_k = d_k;
  g1.pos0 = pos0;
  g1.rope = rope;
  if (cu != nullptr) {
    g1.cu = cu;
    g1.n_cu = n_cu;
    g1.pos_max = (int)max_pos;
  }
  e = launch_project_gemm(g1, dtype, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;

  GemmProblem g2 = g1;
  g2.A = h_D;
  g2.K = d_down;
  g2.a_type = bf ? kF16 : kF32;
  g2.nseg = 2;
  g2.seg[0] = GemmSeg{fK, K_glob, hd, kHead, 1};
  g2.seg[1] = GemmSeg{fV, V_glob, hd, kHeadT, 0};
  e = launch_project_gemm(g2, dtype, stream);
  return hip_status(e);
}

dar_status dar_project(const void* h, const void* W_down, const void* W_up, const void* W_Q,
                       const void* W_K, const void* W_V, const void* W_upK, const void* W_upV,
                       int B, int N, int d, int d_down, int heads, int d_k, int pos0,
                       float rope_base, dar_dtype dtype, void* Q, void* K_loc, void* V_loc,
                       void* h_D, void* K_glob, void* V_glob, void* workspace,
                       size_t* workspace_bytes, hipStream_t stream) {
  return project_impl(h, W_down, W_up, W_Q, W_K, W_V, W_upK, W_upV, B, N, d, d_down, heads, d_k,
                      pos0, rope_base, dtype, Q, K_loc, V_loc, h_D, K_glob, V_glob, workspace,
                      workspace_bytes, stream, 0);
}

dar_status dar_project_sigmoid(const void* h, const void* W_down, const void* W_up,
                               const void* W_Q, const void* W_K, const void* W_V,
                               const void* W_upK, const void* W_upV, int B, int N, int d,
                               int d_down, int heads, int d_k, int pos0, float rope_base,
                               dar_dtype dtype, void* Q, void* K_loc, void* V_loc, void* h_D,
                               void* K_glob, void* V_glob, void* workspace,
                               size_t* workspace_bytes, hipStream_t stream) {
  return project_impl(h, W_down, W_up, W_Q, W_K, W_V, W_upK, W_upV, B, N, d, d_down, heads, d_k,
                      pos0, rope_base, dtype, Q, K_loc, V_loc, h_D, K_glob, V_glob, workspace,
                      workspace_bytes, stream, 1);
}

static dar_status attn_prefill_impl(const void* Q, const void* K_loc, const void* V_loc,
                                    const void* K_glob, const void* V_glob, int B, int N,
                                    int heads, int d_k, int w, dar_dtype dtype, void* o,
                                    float* lse, hipStream_t stream, bool launch = true) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || heads < 1 || d_k < 2 || (d_k & 1) || w < 0) return DAR_ERR_INVALID_ARG;
  const void* need[] = {Q, K_loc, V_loc, K_glob, V_glob, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  const size_t sz = es * (size_t)B * N * heads * d_k;
  const Span ins[5] = {{Q, sz}, {K_loc, sz}, {V_loc, sz}, {K_glob, sz}, {V_glob, sz}};
  const Span outs[2] = {{o, sz}, {lse, sizeof(float) * (size_t)B * heads * N}};
  if (!disjoint(outs, lse != nullptr ? 2 : 1, ins, 5)) return DAR_ERR_INVALID_ARG;
  if (!head_supported(d_k)) return DAR_ERR_UNSUPPORTED;
  if ((size_t)B * heads * N * d_k > 0x7fffffffffffL) return DAR_ERR_UNSUPPORTED;
  if (!launch) return DAR_OK;
  PrefillProblem p{Q, K_loc, V_loc, K_glob, V_glob, o, B, N, heads, d_k, w};
  p.lse = lse;
  return hip_status(launch_attn_prefill(p, dtype, stream));
}

dar_status dar_attn_prefill(const void* Q, const void* K_loc, const void* V_loc,
                            const void* K_glob, const void* V_glob, int B, int N, int heads,
                            int d_k, int w, dar_dtype dtype, void* o, void* workspace,
                            size_t* workspace_bytes, hipStream_t stream) {
  if (workspace == nullptr && workspace_bytes != nullptr) {
    // size query: validate, then report that no workspace is needed
    const dar_status st = attn_prefill_impl(Q, K_loc, V_loc, K_glob, V_glob, B, N, heads, d_k,
                                            w, dtype, o, nullptr, stream, /*launch=*/false);
    if (st == DAR_OK) *workspace_bytes = 0;
    return st;
  }
  return attn_prefill_impl(Q, K_loc, V_loc, K_glob, V_glob, B, N, heads, d_k, w, dtype, o,
                           nullptr, stream);
}

dar_status dar_pack_weight(const void* W, int rows, int cols, dar_dtype dtype, void* W_packed,
                           hipStream_t stream) {
  if (!dtype_ok(dtype) || rows < 1 || cols < 1 || !aligned16(W) || !aligned16(W_packed))
    return DAR_ERR_INVALID_ARG;
  const size_t bytes = elem_size(dtype) * (size_t)rows * cols;
  if (overlap(Span{W, bytes}, Span{W_packed, bytes})) return DAR_ERR_INVALID_ARG;
  if (rows > 64 * 65535 || cols > 64 * 65535) return DAR_ERR_UNSUPPORTED;
  return hip_status(launch_pack_weight(W, rows, cols, (int)elem_size(dtype), W_packed, stream));
}

dar_status dar_attn_prefill_lse(const void* Q, const void* K_loc, const void* V_loc,
                                const void* K_glob, const void* V_glob, int B, int N, int heads,
                                int d_k, int w, dar_dtype dtype, void* o, float* lse,
                                hipStream_t stream) {
  if (!aligned16(lse)) return DAR_ERR_INVALID_ARG;
  return attn_prefill_impl(Q, K_loc, V_loc, K_glob, V_glob, B, N, heads, d_k, w, dtype, o, lse,
                           stream);
}

dar_status dar_project_varlen(const void* h, const void* W_down, const void* W_up,
                              const void* W_Q, const void* W_K, const void* W_V,
                              const void* W_upK, const void* W_upV, const int* cu_seqlens, int B,
                              int T, int max_len, int d, int d_down, int heads, int d_k,
                              float rope_base, dar_dtype dtype, void* Q, void* K_loc,
                              void* V_loc, void* h_D, void* K_glob, void* V_glob,
                              void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype) || B < 1 || T < 1 || max_len < 1 || max_len > T ||
      ((uintptr_t)cu_seqlens & 3u) != 0 || cu_seqlens == nullptr)
    return DAR_ERR_INVALID_ARG;
  const Span cs{cu_seqlens, sizeof(int) * ((size_t)B + 1)};
  const Span outs[6] = {{Q, 2 * (size_t)T * heads * d_k},     {K_loc, 2 * (size_t)T * heads * d_k},
                        {V_loc, 2 * (size_t)T * heads * d_k}, {h_D, 2 * (size_t)T * d_down},
                        {K_glob, 2 * (size_t)T * heads * d_k}, {V_glob, 2 * (size_t)T * heads * d_k}};
  for (const Span& x : outs)
    if (overlap(cs, x)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  return project_impl(h, W_down, W_up, W_Q, W_K, W_V, W_upK, W_upV, 1, T, d, d_down, heads, d_k, 0,
                      rope_base, dtype, Q, K_loc, V_loc, h_D, K_glob, V_glob, workspace,
                      workspace_bytes, stream, 0, cu_seqlens, B, max_len);
}

dar_status dar_attn_prefill_varlen(const void* Q, const void* K_loc, const void* V_loc,
                                   const void* K_glob, const void* V_glob, const int* cu_seqlens,
                                   int B, int T, int max_len, int heads, int d_k, int w,
                                   dar_dtype dtype, void* o, hipStream_t stream) {
  if (!dtype_ok(dtype) || B < 1 || T < 1 || max_len < 1 || max_len > T || heads < 1 || d_k < 2 ||
      (d_k & 1) || w < 0 || cu_seqlens == nullptr || ((uintptr_t)cu_seqlens & 3u) != 0)
    return DAR_ERR_INVALID_ARG;
  const void* need[] = {Q, K_loc, V_loc, K_glob, V_glob, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const size_t sz = 2 * (size_t)T * heads * d_k;
  const Span ins[6] = {{Q, sz},      {K_loc, sz}, {V_loc, sz},
                       {K_glob, sz}, {V_glob, sz}, {cu_seqlens, sizeof(int) * ((size_t)B + 1)}};
  const Span outs[1] = {{o, sz}};
  if (!disjoint(outs, 1, ins, 6)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!head_supported(d_k)) return DAR_ERR_UNSUPPORTED;
  if ((size_t)T * heads * d_k > 0x7fffffffffffL) return DAR_ERR_UNSUPPORTED;
  PrefillProblem p{Q, K_loc, V_loc, K_glob, V_glob, o, B, max_len, heads, d_k, w};
  p.cu = cu_seqlens;
  p.T = T;
  return hip_status(launch_attn_prefill(p, dtype, stream));
}

dar_status dar_attn_prefill_backward(const void* Q, const void* K_loc, const void* V_loc,
                                     const void* K_glob, const void* V_glob, const void* o,
                                     const void* dO, const float* lse, int B, int N, int heads,
                                     int d_k, int w, dar_dtype dtype, float* dQ, float* dK_loc,
                                     float* dV_loc,
                                     float* dK_glob, float* dV_glob, void* workspace,
                                     size_t* workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || heads < 1 || d_k < 2 || (d_k & 1) || w < 0) return DAR_ERR_INVALID_ARG;
  const void* need[] = {Q, K_loc, V_loc, K_glob, V_glob, o, dO, dQ, dK_loc, dV_loc, dK_glob,
                        dV_glob};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const size_t n_el = (size_t)B * N * heads * d_k;
  const size_t sz = elem_size(dtype) * n_el, gz = sizeof(float) * n_el;
  if (lse != nullptr && ((uintptr_t)lse & 3u)) return DAR_ERR_INVALID_ARG;
  const Span ins[8] = {{Q, sz},      {K_loc, sz}, {V_loc, sz}, {K_glob, sz},
                       {V_glob, sz}, {o, sz},     {dO, sz},    {lse, sizeof(float) * n_el / d_k}};
  const Span outs[5] = {{dQ, gz}, {dK_loc, gz}, {dV_loc, gz}, {dK_glob, gz}, {dV_glob, gz}};
  if (!disjoint(outs, 5, ins, 8)) return DAR_ERR_INVALID_ARG;
  if (!head_supported(d_k)) return DAR_ERR_UNSUPPORTED;
  if (n_el > 0x7fffffffffffL || (size_t)B * heads > 0x7fffffff / ((size_t)N + 63))
    return DAR_ERR_UNSUPPORTED;
  const size_t need_bytes = attn_backward_workspace_bytes(B, N, heads);
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& x : ins)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
    for (const Span& x : outs)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
  }
  BwdProblem p{};
  p.Q = Q;
  p.K_loc = K_loc;
  p.V_loc = V_loc;
  p.K_glob = K_glob;
  p.V_glob = V_glob;
  p.o = o;
  p.dO = dO;
  p.lse_in = lse;
  p.dQ = dQ;
  p.dK_loc = dK_loc;
  p.dV_loc = dV_loc;
  p.dK_glob = dK_glob;
  p.dV_glob = dV_glob;
  p.lse = (float*)workspace;
  p.Dd = (float*)((char*)workspace + need_bytes / 2);
  p.B = B;
  p.N = N;
  p.H = heads;
  p.d_k = d_k;
  p.w = w;
  return hip_status(launch_attn_backward(p, dtype, stream));
}

// Decode append, uniform (pos_arr == nullptr: every sequence at position pos)
// or ragged (pos_arr: device int32[B], sequence b at pos_arr[b] < cap).
static dar_status decode_append_impl(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, int B, int d, int d_down,
                                     int heads, int d_k, int pos, const int* pos_arr, int w,
                                     int cap, float rope_base, dar_dtype dtype, void* q,
                                     void* K_win, void* V_win, void* h_D, void* workspace,
                                     size_t* workspace_bytes, hipStream_t stream, int act) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1) || pos < 0 || w < 0 ||
      cap < 1)
    return DAR_ERR_INVALID_ARG;
  if (pos >= cap || !(rope_base > 1.0f)) return DAR_ERR_INVALID_ARG;
  if (pos_arr != nullptr && ((uintptr_t)pos_arr & 3u)) return DAR_ERR_INVALID_ARG;
  const void* need[] = {h, W_down, W_Q, W_K, W_V, q, h_D};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_win) || !aligned16(V_win))) return DAR_ERR_INVALID_ARG;
  const int hd = heads * d_k;
  const size_t es = elem_size(dtype);
  const Span ins[6] = {{h, es * B * (size_t)d}, {W_down, es * d * (size_t)d_down},
                       {W_Q, es * d * (size_t)hd}, {W_K, es * d * (size_t)hd},
                       {W_V, es * d * (size_t)hd}, {pos_arr, sizeof(int) * (size_t)B}};
  const Span outs[4] = {{q, es * B * (size_t)hd},
                        {K_win, w > 0 ? es * B * (size_t)hd * w : 0},
                        {V_win, w > 0 ? es * B * (size_t)hd * w : 0},
                        {h_D, es * B * (size_t)cap * d_down}};
  if (!disjoint(outs, 4, ins, 6)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!head_supported(d_k) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;
  // ragged positions are only known on the device: tables cover the cache
  const int max_pos = pos_arr != nullptr ? cap - 1 : pos;
  const size_t need_bytes = rope_table_bytes(d_k, max_pos);
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& sp : ins)
      if (overlap(ws, sp)) return DAR_ERR_INVALID_ARG;
    for (const Span& sp : outs)
      if (overlap(ws, sp)) return DAR_ERR_INVALID_ARG;
  }
  float2* lo = (float2*)workspace;
  float2* hi = lo + 64 * (d_k / 2);
  hipError_t e = launch_rope_tables(lo, hi, d_k, max_pos, rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  // One GEMM over the B new tokens (one per sequence, at position pos or
  // pos_arr[b]): q at [b, head, 0, t]; k, v into ring slot pos mod w; h^D into
  // row pos.
  GemmProblem g{};
  g.A = h;
  g.M = B;
  g.K = d;
  g.a_type = kBF16;
  g.b_type = kBF16;
  g.out_type = kBF16;
  g.n_seq = 1;
  g.heads = heads;
  g.d_k = d_k;
  g.pos0 = pos;
  g.rope = RopeTab{lo, hi, d_k / 2};
  g.row_pos = pos_arr;
  g.pos_max = max_pos;
  int ns = 0;
  g.seg[ns++] = GemmSeg{W_Q, q, hd, kHead, 1, 1, 0, kPosFixed};
  if (w > 0) {
    g.seg[ns++] = GemmSeg{W_K, K_win, hd, kHead, 1, w, pos % w, kPosRing};
    g.seg[ns++] = GemmSeg{W_V, V_win, hd, kHead, 0, w, pos % w, kPosRing};
  }
  g.seg[ns] = GemmSeg{W_down, h_D, d_down, kRowMajor, 0, cap, pos, kPosRow};
  g.seg[ns++].act = act;
  g.nseg = ns;
  return hip_status(launch_project_gemm(g, dtype, stream));
}

dar_status dar_decode_append(const void* h, const void* W_down, const void* W_Q, const void* W_K,
                             const void* W_V, int B, int d, int d_down, int heads, int d_k,
                             int pos, int w, int cap, float rope_base, dar_dtype dtype, void* q,
                             void* K_win, void* V_win, void* h_D, void* workspace,
                             size_t* workspace_bytes, hipStream_t stream) {
  return decode_append_impl(h, W_down, W_Q, W_K, W_V, B, d, d_down, heads, d_k, pos, nullptr, w,
                            cap, rope_base, dtype, q, K_win, V_win, h_D, workspace,
                            workspace_bytes, stream, 0);
}

dar_status dar_decode_append_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, int B, int d, int d_down,
                                     int heads, int d_k, int pos, int w, int cap, float rope_base,
                                     dar_dtype dtype, void* q, void* K_win, void* V_win, void* h_D,
                                     void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream) {
  return decode_append_impl(h, W_down, W_Q, W_K, W_V, B, d, d_down, heads, d_k, pos, nullptr, w,
                            cap, rope_base, dtype, q, K_win, V_win, h_D, workspace,
                            workspace_bytes, stream, 1);
}

dar_status dar_decode_append_varlen(const void* h, const void* W_down, const void* W_Q,
                                    const void* W_K, const void* W_V, int B, int d, int d_down,
                                    int heads, int d_k, const int* pos, int w, int cap,
                                    float rope_base, dar_dtype dtype, void* q, void* K_win,
                                    void* V_win, void* h_D, void* workspace,
                                    size_t* workspace_bytes, hipStream_t stream) {
  if (pos == nullptr) return DAR_ERR_INVALID_ARG;
  return decode_append_impl(h, W_down, W_Q, W_K, W_V, B, d, d_down, heads, d_k, 0, pos, w, cap,
                            rope_base, dtype, q, K_win, V_win, h_D, workspace, workspace_bytes,
                            stream, 0);
}

dar_status dar_decode_append_varlen_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                            const void* W_K, const void* W_V, int B, int d,
                                            int d_down, int heads, int d_k, const int* pos, int w,
                                            int cap, float rope_base, dar_dtype dtype, void* q,
                                            void* K_win, void* V_win, void* h_D, void* workspace,
                                            size_t* workspace_bytes, hipStream_t stream) {
  if (pos == nullptr) return DAR_ERR_INVALID_ARG;
  return decode_append_impl(h, W_down, W_Q, W_K, W_V, B, d, d_down, heads, d_k, 0, pos, w, cap,
                            rope_base, dtype, q, K_win, V_win, h_D, workspace, workspace_bytes,
                            stream, 1);
}

static dar_status cache_from_prefill_impl(const void* h_D, const void* K_loc, const void* V_loc,
                                          int B, int N, const int* lens, int heads, int d_k,
                                          int d_down, int w, int cap, dar_dtype dtype,
                                          void* h_D_cache, void* K_win, void* V_win,
                                          hipStream_t stream) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_down < 1 || w < 0 || cap < N)
    return DAR_ERR_INVALID_ARG;
  if (lens != nullptr && ((uintptr_t)lens & 3u)) return DAR_ERR_INVALID_ARG;
  if (!aligned16(h_D) || !aligned16(h_D_cache)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_loc) || !aligned16(V_loc) || !aligned16(K_win) || !aligned16(V_win)))
    return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k;
  const Span ins[4] = {{h_D, 2 * (size_t)B * N * d_down},
                       {w > 0 ? K_loc : nullptr, 2 * (size_t)B * N * hd},
                       {w > 0 ? V_loc : nullptr, 2 * (size_t)B * N * hd},
                       {lens, sizeof(int) * (size_t)B}};
  const Span outs[3] = {{h_D_cache, 2 * (size_t)B * cap * d_down},
                        {w > 0 ? K_win : nullptr, 2 * (size_t)B * w * hd},
                        {w > 0 ? V_win : nullptr, 2 * (size_t)B * w * hd}};
  if (!disjoint(outs, 3, ins, 4)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!head_supported(d_k) || d_down % 8) return DAR_ERR_UNSUPPORTED;
  return hip_status(launch_cache_from_prefill(h_D, K_loc, V_loc, B, N, heads, d_k, d_down, w,
                                              cap, h_D_cache, K_win, V_win, stream, lens));
}

dar_status dar_cache_from_prefill(const void* h_D, const void* K_loc, const void* V_loc, int B,
                                  int N, int heads, int d_k, int d_down, int w, int cap,
                                  dar_dtype dtype, void* h_D_cache, void* K_win, void* V_win,
                                  hipStream_t stream) {
  return cache_from_prefill_impl(h_D, K_loc, V_loc, B, N, nullptr, heads, d_k, d_down, w, cap,
                                 dtype, h_D_cache, K_win, V_win, stream);
}

dar_status dar_cache_from_prefill_varlen(const void* h_D, const void* K_loc, const void* V_loc,
                                         int B, int N, const int* lens, int heads, int d_k,
                                         int d_down, int w, int cap, dar_dtype dtype,
                                         void* h_D_cache, void* K_win, void* V_win,
                                         hipStream_t stream) {
  if (lens == nullptr) return DAR_ERR_INVALID_ARG;
  return cache_from_prefill_impl(h_D, K_loc, V_loc, B, N, lens, heads, d_k, d_down, w, cap,
                                 dtype, h_D_cache, K_win, V_win, stream);
}

dar_status dar_cache_from_prefill_packed(const void* h_D, const void* K_loc, const void* V_loc,
                                         const int* cu_seqlens, int B, int T, int max_len,
                                         int heads, int d_k, int d_down, int w, int cap,
                                         dar_dtype dtype, void* h_D_cache, void* K_win,
                                         void* V_win, hipStream_t stream) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || T < 1 || max_len < 1 || max_len > T || heads < 1 || d_k < 2 || (d_k & 1) ||
      d_down < 1 || w < 0 || cap < max_len || cu_seqlens == nullptr ||
      ((uintptr_t)cu_seqlens & 3u) != 0)
    return DAR_ERR_INVALID_ARG;
  if (!aligned16(h_D) || !aligned16(h_D_cache)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_loc) || !aligned16(V_loc) || !aligned16(K_win) || !aligned16(V_win)))
    return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k;
  const Span ins[4] = {{h_D, 2 * (size_t)T * d_down},
                       {w > 0 ? K_loc : nullptr, 2 * (size_t)T * hd},
                       {w > 0 ? V_loc : nullptr, 2 * (size_t)T * hd},
                       {cu_seqlens, sizeof(int) * ((size_t)B + 1)}};
  const Span outs[3] = {{h_D_cache, 2 * (size_t)B * cap * d_down},
                        {w > 0 ? K_win : nullptr, 2 * (size_t)B * w * hd},
                        {w > 0 ? V_win : nullptr, 2 * (size_t)B * w * hd}};
  if (!disjoint(outs, 3, ins, 4)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!head_supported(d_k) || d_down % 8 || (long)B * heads > 0x7fffffffL)
    return DAR_ERR_UNSUPPORTED;
  return hip_status(launch_cache_from_packed(h_D, K_loc, V_loc, cu_seqlens, B, T, max_len, heads,
                                             d_k, d_down, w, cap, h_D_cache, K_win, V_win,
                                             stream));
}

static dar_status prefill_chunk_impl(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, const void* W_upK,
                                     const void* W_upV, int B, int C, int d, int d_down, int heads,
                                     int d_k, int p0, int w, int cap, float rope_base,
                                     dar_dtype dtype, void* h_D_cache, void* K_win, void* V_win,
                                     void* o, void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream, int act) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || C < 1 || d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1) || p0 < 0 ||
      w < 0 || cap < 1 || (long)p0 + C > cap || !(rope_base > 1.f) || workspace_bytes == nullptr)
    return DAR_ERR_INVALID_ARG;
  const void* need[] = {h, W_down, W_Q, W_K, W_V, W_upK, W_upV, h_D_cache, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_win) || !aligned16(V_win))) return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k;
  const Span ins[7] = {{h, 2 * (size_t)B * C * d},       {W_down, 2 * (size_t)d * d_down},
                       {W_Q, 2 * (size_t)d * hd},         {W_K, 2 * (size_t)d * hd},
                       {W_V, 2 * (size_t)d * hd},         {W_upK, 2 * (size_t)d_down * hd},
                       {W_upV, 2 * (size_t)d_down * hd}};
  const Span outs[4] = {{h_D_cache, 2 * (size_t)B * cap * d_down},
                        {w > 0 ? K_win : nullptr, 2 * (size_t)B * w * hd},
                        {w > 0 ? V_win : nullptr, 2 * (size_t)B * w * hd},
                        {o, 2 * (size_t)B * C * hd}};
  if (!disjoint(outs, 4, ins, 7)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!head_supported(d_k) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;

  // Positions: the chunk is p0 .. N-1.  Global keys 0 .. N-1 are rebuilt from
  // the latents; local keys that a chunk query can use are p0-w+1 .. N-1
  // (the ring's, then the chunk's own).  The local arrays start at loc0, that
  // position rounded down to a multiple of 64 (rows below p0-w+1 hold zeros
  // and are never kept), so that their key tiles are whole.
  const int N = p0 + C;
  const int loc0 = w > 0 ? std::max(0, p0 - (w - 1)) / 64 * 64 : N;
  const int nloc = N - loc0;
  const size_t rope_bytes = rope_table_bytes(d_k, N - 1);
  const size_t q_bytes = round256(2 * (size_t)B * hd * C);
  const size_t hdc_bytes = round256(2 * (size_t)B * C * d_down);
  const size_t glob_bytes = round256(2 * (size_t)B * hd * N);
  const size_t loc_bytes = round256(2 * (size_t)B * hd * nloc);
  const size_t need_bytes = rope_bytes + q_bytes + hdc_bytes + 2 * glob_bytes + 2 * loc_bytes;
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& sp : ins)
      if (overlap(ws, sp)) return DAR_ERR_INVALID_ARG;
    for (const Span& sp : outs)
      if (overlap(ws, sp)) return DAR_ERR_INVALID_ARG;
  }
  char* wsp = (char*)workspace;
  float2* lo = (float2*)wsp;
  float2* hi = lo + 64 * (d_k / 2);
  char* cur = wsp + rope_bytes;
  void* Qc = cur;
  cur += q_bytes;
  void* hDc = cur;
  cur += hdc_bytes;
  void* Kg = cur;
  cur += glob_bytes;
  void* Vg = cur;
  cur += glob_bytes;
  void* Kl = cur;
  cur += loc_bytes;
  void* Vl = cur;
  const RopeTab rope{lo, hi, d_k / 2};

  hipError_t e = launch_rope_tables(lo, hi, d_k, N - 1, rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  // 1. the chunk's projections: q, local k / v (after the ring's rows of the
  //    local arrays), h^D (fp16, then into the latent cache)
  GemmProblem g1{};
  g1.A = h;
  g1.M = B * C;
  g1.K = d;
  g1.a_type = kBF16;
  g1.b_type = kBF16;
  g1.out_type = kF16;
  g1.n_seq = C;
  g1.heads = heads;
  g1.d_k = d_k;
  g1.pos0 = p0;
  g1.rope = rope;
  int ns = 0;
  g1.seg[ns++] = GemmSeg{W_Q, Qc, (int)hd, kHead, 1};
  if (w > 0) {
    g1.seg[ns++] = GemmSeg{W_K, Kl, (int)hd, kHead, 1, nloc, p0 - loc0};
    g1.seg[ns++] = GemmSeg{W_V, Vl, (int)hd, kHeadT, 0, nloc, p0 - loc0};
  }
  g1.seg[ns] = GemmSeg{W_down, hDc, d_down, kRowMajor, 0};
  g1.seg[ns++].act = act;
  g1.nseg = ns;
  e = launch_project_gemm(g1, dtype, stream);
  if (e == hipSuccess) e = launch_latent_cast(hDc, B, C, d_down, cap, p0, h_D_cache, stream);
  // 2. the prefix's ring rows into the local arrays
  if (e == hipSuccess)
    e = launch_ring_to_local(K_win, V_win, B, heads, d_k, w, loc0, p0, nloc, Kl, Vl, stream);
  // 3. global keys / values of the prefix from the latent cache, then of the
  //    chunk from its fp16 h^D.  The prefix is one GEMM over every sequence
  //    (cache rows cap apart) while the cache is under 2 GiB, else one per
  //    sequence.
  const bool one = 2 * (size_t)B * cap * d_down <= (size_t)0x7ffffff0;
  for (int b = 0; b < (one ? 1 : B) && p0 > 0 && e == hipSuccess; ++b) {
    GemmProblem g2{};
    g2.A = (const char*)h_D_cache + 2 * (size_t)b * cap * d_down;
    g2.M = one ? B * p0 : p0;
    g2.a_ld_seq = one ? cap : 0;
    g2.K = d_down;
    g2.a_type = kBF16;
    g2.b_type = kBF16;
    g2.out_type = kF16;
    g2.n_seq = p0;
    g2.heads = heads;
    g2.d_k = d_k;
    g2.pos0 = 0;
    g2.rope = rope;
    g2.nseg = 2;
    g2.seg[0] = GemmSeg{W_upK, (char*)Kg + 2 * (size_t)b * hd * N, (int)hd, kHead, 1, N, 0};
    g2.seg[1] = GemmSeg{W_upV, (char*)Vg + 2 * (size_t)b * hd * N, (int)hd, kHeadT, 0, N, 0};
    e = launch_project_gemm(g2, dtype, stream);
  }
  if (e == hipSuccess) {
    GemmProblem g3{};
    g3.A = hDc;
    g3.M = B * C;
    g3.K = d_down;
    g3.a_type = kF16;
    g3.b_type = kBF16;
    g3.out_type = kF16;
    g3.n_seq = C;
    g3.heads = heads;
    g3.d_k = d_k;
    g3.pos0 = p0;
    g3.rope = rope;
    g3.nseg = 2;
    g3.seg[0] = GemmSeg{W_upK, Kg, (int)hd, kHead, 1, N, p0};
    g3.seg[1] = GemmSeg{W_upV, Vg, (int)hd, kHeadT, 0, N, p0};
    e = launch_project_gemm(g3, dtype, stream);
  }
  // 4. attention of the chunk's queries over positions 0 .. N-1
  if (e == hipSuccess) {
    PrefillProblem pp{};
    pp.Q = Qc;
    pp.K_loc = Kl;
    pp.V_loc = Vl;
    pp.K_glob = Kg;
    pp.V_glob = Vg;
    pp.o = o;
    pp.B = B;
    pp.N = N;
    pp.H = heads;
    pp.d_k = d_k;
    pp.w = w;
    pp.q0 = p0;
    pp.loc0 = loc0;
    e = launch_attn_prefill(pp, dtype, stream);
  }
  // 5. the ring moves on to positions N-w .. N-1
  if (e == hipSuccess)
    e = launch_ring_fill(Kl, Vl, B, heads, d_k, N, loc0, w, K_win, V_win, stream);
  return hip_status(e);
}

dar_status dar_prefill_chunk(const void* h, const void* W_down, const void* W_Q, const void* W_K,
                             const void* W_V, const void* W_upK, const void* W_upV, int B, int C,
                             int d, int d_down, int heads, int d_k, int p0, int w, int cap,
                             float rope_base, dar_dtype dtype, void* h_D_cache, void* K_win,
                             void* V_win, void* o, void* workspace, size_t* workspace_bytes,
                             hipStream_t stream) {
  return prefill_chunk_impl(h, W_down, W_Q, W_K, W_V, W_upK, W_upV, B, C, d, d_down, heads, d_k,
                            p0, w, cap, rope_base, dtype, h_D_cache, K_win, V_win, o, workspace,
                            workspace_bytes, stream, 0);
}

dar_status dar_prefill_chunk_sigmoid(const void* h, const void* W_down, const void* W_Q,
                                     const void* W_K, const void* W_V, const void* W_upK,
                                     const void* W_upV, int B, int C, int d, int d_down, int heads,
                                     int d_k, int p0, int w, int cap, float rope_base,
                                     dar_dtype dtype, void* h_D_cache, void* K_win, void* V_win,
                                     void* o, void* workspace, size_t* workspace_bytes,
                                     hipStream_t stream) {
  return prefill_chunk_impl(h, W_down, W_Q, W_K, W_V, W_upK, W_upV, B, C, d, d_down, heads, d_k,
                            p0, w, cap, rope_base, dtype, h_D_cache, K_win, V_win, o, workspace,
                            workspace_bytes, stream, 1);
}

static dar_status attn_decode_impl(const void* q, const void* K_win, const void* V_win,
                                   const void* h_D, const void* W_upK, const void* W_upV, int B,
                                   int ctx_len, const int* ctx_lens, int cap, int heads, int d_k,
                                   int d_down, int w, float rope_base, dar_dtype dtype, void* o,
                                   void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (ctx_lens != nullptr && ((uintptr_t)ctx_lens & 3u)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || ctx_len < 1 || cap < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_down < 1 ||
      w < 0)
    return DAR_ERR_INVALID_ARG;
  if (!(rope_base > 1.0f)) return DAR_ERR_INVALID_ARG;
  const long p_pos = (long)ctx_len - 1;
  const long n_glob = std::max(0L, p_pos - w + 1);
  if (n_glob > cap) return DAR_ERR_INVALID_ARG;
  const void* need[] = {q, h_D, W_upK, W_upV, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_win) || !aligned16(V_win))) return DAR_ERR_INVALID_ARG;
  const int hd = heads * d_k;
  const size_t es = elem_size(dtype);
  const Span ins[7] = {{q, es * B * hd},
                       {K_win, w > 0 ? es * B * hd * (size_t)w : 0},
                       {V_win, w > 0 ? es * B * hd * (size_t)w : 0},
                       {h_D, es * B * (size_t)cap * d_down},
                       {W_upK, es * d_down * hd},
                       {W_upV, es * d_down * hd},
                       {ctx_lens, sizeof(int) * (size_t)B}};
  const Span outs[1] = {{o, es * B * hd}};
  if (!disjoint(outs, 1, ins, 7)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!decode_supported(d_k, d_down) || hd % 64) return DAR_ERR_UNSUPPORTED;

  DecodeProblem p{};
  p.q = q;
  p.K_win = K_win;
  p.V_win = V_win;
  p.h_D = h_D;
  p.W_upK = W_upK;
  p.W_upV = W_upV;
  p.o = o;
  p.B = B;
  p.ctx = ctx_len;
  p.cap = cap;
  p.H = heads;
  p.d_k = d_k;
  p.d_down = d_down;
  p.w = w;
  p.ctx_lens = ctx_lens;
  const size_t rope_bytes = rope_table_bytes(d_k, std::max(0L, n_glob - 1));
  const size_t need_bytes = rope_bytes + decode_workspace_bytes(p);
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& s : ins)
      if (overlap(ws, s)) return DAR_ERR_INVALID_ARG;
    if (overlap(ws, outs[0])) return DAR_ERR_INVALID_ARG;
  }
  char* wsp = (char*)workspace;
  float2* lo = (float2*)wsp;
  float2* hi = lo + 64 * (d_k / 2);
  hipError_t e = launch_rope_tables(lo, hi, d_k, std::max(0L, n_glob - 1), rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  p.rope = RopeTab{lo, hi, d_k / 2};
  p.ws = wsp + rope_bytes;
  return hip_status(launch_attn_decode(p, stream));
}

dar_status dar_attn_decode(const void* q, const void* K_win, const void* V_win, const void* h_D,
                           const void* W_upK, const void* W_upV, int B, int ctx_len, int cap,
                           int heads, int d_k, int d_down, int w, float rope_base,
                           dar_dtype dtype, void* o, void* workspace, size_t* workspace_bytes,
                           hipStream_t stream) {
  return attn_decode_impl(q, K_win, V_win, h_D, W_upK, W_upV, B, ctx_len, nullptr, cap, heads,
                          d_k, d_down, w, rope_base, dtype, o, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- decoupled RoPE
static bool drope_shape_ok(int d_k, int d_R) { return (d_k == 64 || d_k == 128) && d_R == 64; }

dar_status dar_project_drope(const void* h, const void* W_down, const void* W_up, const void* W_Q,
                             const void* W_K, const void* W_V, const void* W_QR, const void* W_KR,
                             const void* W_upK, const void* W_upV, int B, int N, int d,
                             int d_down, int heads, int d_k, int d_R, int pos0, float rope_base,
                             dar_dtype dtype, void* QC, void* QR, void* K_loc, void* V_loc,
                             void* h_D, void* K_glob, void* V_glob, void* KR, void* workspace,
                             size_t* workspace_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_R < 2 ||
      (d_R & 1) || pos0 < 0 || !(rope_base > 1.0f) || (long)pos0 + N - 1 > 0x7fffffffL)
    return DAR_ERR_INVALID_ARG;
  const bool have_fold = (W_upK != nullptr) || (W_upV != nullptr);
  if (have_fold && (!aligned16(W_upK) || !aligned16(W_upV))) return DAR_ERR_INVALID_ARG;
  if (!have_fold && !aligned16(W_up)) return DAR_ERR_INVALID_ARG;
  const void* need[] = {h, W_down, W_Q, W_K, W_V, W_QR, W_KR, QC, QR, K_loc, V_loc, h_D,
                        K_glob, V_glob, KR};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k, hr = (size_t)heads * d_R, M = (size_t)B * N;
  const size_t es = elem_size(dtype);
  const Span ins[10] = {{h, es * M * d},         {W_down, es * d * d_down},
                        {W_Q, es * d * hd},      {W_K, es * d * hd},
                        {W_V, es * d * hd},      {W_QR, es * d * hr},
                        {W_KR, es * d * d_R},    {have_fold ? nullptr : W_up, es * d_down * d},
                        {W_upK, es * d_down * hd}, {W_upV, es * d_down * hd}};
  const Span outs[8] = {{QC, es * M * hd},     {QR, es * M * hr},     {K_loc, es * M * hd},
                        {V_loc, es * M * hd},  {h_D, es * M * d_down}, {K_glob, es * M * hd},
                        {V_glob, es * M * hd}, {KR, es * M * d_R}};
  if (!disjoint(outs, 8, ins, 10)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!drope_shape_ok(d_k, d_R) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;
  const long max_pos = (long)pos0 + N - 1;
  const size_t rope_bytes = rope_table_bytes(d_R, max_pos);
  const size_t fold_bytes = have_fold ? 0 : 2 * round256(es * d_down * hd);
  const size_t need_bytes = rope_bytes + fold_bytes;
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& x : ins)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
    for (const Span& x : outs)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
  }
  char* wsp = (char*)workspace;
  float2* lo = (float2*)wsp;
  float2* hi = lo + 64 * (d_R / 2);
  hipError_t e = launch_rope_tables(lo, hi, d_R, max_pos, rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  const void* fK = W_upK;
  const void* fV = W_upV;
  if (!have_fold) {
    void* k_out = wsp + rope_bytes;
    void* v_out = wsp + rope_bytes + round256(es * d_down * hd);
    e = launch_fold(W_up, W_K, k_out, d, d_down, (int)hd, dtype, stream);
    if (e == hipSuccess) e = launch_fold(W_up, W_V, v_out, d, d_down, (int)hd, dtype, stream);
    if (e != hipSuccess) return DAR_ERR_HIP;
    fK = k_out;
    fV = v_out;
  }
  const RopeTab rope{lo, hi, d_R / 2};
  // content parts, values and the latent (no rotation)
  GemmProblem g1{};
  g1.A = h;
  g1.M = (int)M;
  g1.K = d;
  g1.a_type = kBF16;
  g1.b_type = kBF16;
  g1.out_type = kF16;
  g1.nseg = 4;
  g1.seg[0] = GemmSeg{W_Q, QC, (int)hd, kHead, 0};
  g1.seg[1] = GemmSeg{W_K, K_loc, (int)hd, kHead, 0};
  g1.seg[2] = GemmSeg{W_V, V_loc, (int)hd, kHeadT, 0};
  g1.seg[3] = GemmSeg{W_down, h_D, d_down, kRowMajor, 0};
  g1.n_seq = N;
  g1.heads = heads;
  g1.d_k = d_k;
  g1.pos0 = pos0;
  g1.rope = rope;
  e = launch_project_gemm(g1, dtype, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  // rotary parts: the heads' queries and the one shared key
  GemmProblem gr = g1;
  gr.nseg = 2;
  gr.d_k = d_R;
  gr.seg[0] = GemmSeg{W_QR, QR, (int)hr, kHead, 1};
  gr.seg[1] = GemmSeg{W_KR, KR, d_R, kHead, 1};
  gr.seg[1].heads = 1;
  e = launch_project_gemm(gr, dtype, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  // global content keys and values from h^D through the folded weights
  GemmProblem g2 = g1;
  g2.A = h_D;
  g2.K = d_down;
  g2.a_type = kF16;
  g2.nseg = 2;
  g2.seg[0] = GemmSeg{fK, K_glob, (int)hd, kHead, 0};
  g2.seg[1] = GemmSeg{fV, V_glob, (int)hd, kHeadT, 0};
  return hip_status(launch_project_gemm(g2, dtype, stream));
}

dar_status dar_attn_prefill_drope(const void* QC, const void* QR, const void* K_loc,
                                  const void* V_loc, const void* K_glob, const void* V_glob,
                                  const void* KR, int B, int N, int heads, int d_k, int d_R, int w,
                                  dar_dtype dtype, void* o, hipStream_t stream) {
  if (!dtype_ok(dtype)) return DAR_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_R < 2 || (d_R & 1) || w < 0)
    return DAR_ERR_INVALID_ARG;
  const void* need[] = {QC, QR, K_loc, V_loc, K_glob, V_glob, KR, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype), n = (size_t)B * N * heads;
  const Span ins[7] = {{QC, es * n * d_k},     {QR, es * n * d_R},     {K_loc, es * n * d_k},
                       {V_loc, es * n * d_k},  {K_glob, es * n * d_k}, {V_glob, es * n * d_k},
                       {KR, es * (size_t)B * N * d_R}};
  const Span outs[1] = {{o, es * n * d_k}};
  if (!disjoint(outs, 1, ins, 7)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!drope_shape_ok(d_k, d_R)) return DAR_ERR_UNSUPPORTED;
  if (n * (d_k + d_R) > 0x7fffffffffffL) return DAR_ERR_UNSUPPORTED;
  PrefillProblem p{QC, K_loc, V_loc, K_glob, V_glob, o, B, N, heads, d_k, w};
  p.QR = QR;
  p.KR = KR;
  p.d_R = d_R;
  return hip_status(launch_attn_prefill(p, dtype, stream));
}

dar_status dar_decode_append_drope(const void* h, const void* W_down, const void* W_Q,
                                   const void* W_K, const void* W_V, const void* W_QR,
                                   const void* W_KR, int B, int d, int d_down, int heads, int d_k,
                                   int d_R, int pos, int w, int cap, float rope_base,
                                   dar_dtype dtype, void* qC, void* qR, void* K_win, void* V_win,
                                   void* h_D, void* KR, void* workspace, size_t* workspace_bytes,
                                   hipStream_t stream) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || d < 1 || d_down < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_R < 2 || (d_R & 1) ||
      pos < 0 || w < 0 || cap < 1 || pos >= cap || !(rope_base > 1.0f))
    return DAR_ERR_INVALID_ARG;
  const void* need[] = {h, W_down, W_Q, W_K, W_V, W_QR, W_KR, qC, qR, h_D, KR};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_win) || !aligned16(V_win))) return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k, hr = (size_t)heads * d_R, es = elem_size(dtype);
  const Span ins[7] = {{h, es * B * (size_t)d},  {W_down, es * d * (size_t)d_down},
                       {W_Q, es * d * hd},       {W_K, es * d * hd},
                       {W_V, es * d * hd},       {W_QR, es * d * hr},
                       {W_KR, es * d * (size_t)d_R}};
  const Span outs[6] = {{qC, es * B * hd},
                        {qR, es * B * hr},
                        {K_win, w > 0 ? es * B * hd * w : 0},
                        {V_win, w > 0 ? es * B * hd * w : 0},
                        {h_D, es * B * (size_t)cap * d_down},
                        {KR, es * B * (size_t)cap * d_R}};
  if (!disjoint(outs, 6, ins, 7)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!drope_shape_ok(d_k, d_R) || d % 64 || d_down % 32 || d_down > 1024 || hd % 64)
    return DAR_ERR_UNSUPPORTED;
  const size_t need_bytes = rope_table_bytes(d_R, pos);
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& x : ins)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
    for (const Span& x : outs)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
  }
  float2* lo = (float2*)workspace;
  float2* hi = lo + 64 * (d_R / 2);
  hipError_t e = launch_rope_tables(lo, hi, d_R, pos, rope_base, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  GemmProblem g{};
  g.A = h;
  g.M = B;
  g.K = d;
  g.a_type = kBF16;
  g.b_type = kBF16;
  g.out_type = kBF16;
  g.n_seq = 1;
  g.heads = heads;
  g.d_k = d_k;
  g.pos0 = pos;
  g.rope = RopeTab{lo, hi, d_R / 2};
  g.pos_max = pos;
  int ns = 0;
  g.seg[ns++] = GemmSeg{W_Q, qC, (int)hd, kHead, 0, 1, 0, kPosFixed};
  if (w > 0) {
    g.seg[ns++] = GemmSeg{W_K, K_win, (int)hd, kHead, 0, w, pos % w, kPosRing};
    g.seg[ns++] = GemmSeg{W_V, V_win, (int)hd, kHead, 0, w, pos % w, kPosRing};
  }
  g.seg[ns++] = GemmSeg{W_down, h_D, d_down, kRowMajor, 0, cap, pos, kPosRow};
  g.nseg = ns;
  e = launch_project_gemm(g, dtype, stream);
  if (e != hipSuccess) return DAR_ERR_HIP;
  GemmProblem gr = g;
  gr.d_k = d_R;
  gr.nseg = 2;
  gr.seg[0] = GemmSeg{W_QR, qR, (int)hr, kHead, 1, 1, 0, kPosFixed};
  gr.seg[1] = GemmSeg{W_KR, KR, d_R, kHead, 1, cap, pos, kPosRow};
  gr.seg[1].heads = 1;
  return hip_status(launch_project_gemm(gr, dtype, stream));
}

dar_status dar_cache_from_prefill_drope(const void* h_D, const void* K_loc, const void* V_loc,
                                        const void* KR, int B, int N, int heads, int d_k,
                                        int d_down, int d_R, int w, int cap, dar_dtype dtype,
                                        void* h_D_cache, void* K_win, void* V_win, void* KR_cache,
                                        hipStream_t stream) {
  if (!dtype_ok(dtype) || B < 1 || N < 1 || cap < N || d_R < 2 || (d_R & 1))
    return DAR_ERR_INVALID_ARG;
  if (!aligned16(KR) || !aligned16(KR_cache)) return DAR_ERR_INVALID_ARG;
  const Span kr_in{KR, 2 * (size_t)B * N * d_R}, kr_out{KR_cache, 2 * (size_t)B * cap * d_R};
  const Span others[5] = {{h_D, 2 * (size_t)B * N * d_down},
                          {h_D_cache, 2 * (size_t)B * cap * d_down},
                          {w > 0 ? K_win : nullptr, 2 * (size_t)B * w * heads * d_k},
                          {w > 0 ? V_win : nullptr, 2 * (size_t)B * w * heads * d_k},
                          {w > 0 ? K_loc : nullptr, 2 * (size_t)B * N * heads * d_k}};
  if (overlap(kr_in, kr_out)) return DAR_ERR_INVALID_ARG;
  for (const Span& x : others)
    if (overlap(kr_out, x) || overlap(kr_in, x)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!drope_shape_ok(d_k, d_R)) return DAR_ERR_UNSUPPORTED;
  // the latent rows and the ring: as for the exact method (content keys)
  const dar_status st = cache_from_prefill_impl(h_D, K_loc, V_loc, B, N, nullptr, heads, d_k,
                                                d_down, w, cap, dtype, h_D_cache, K_win, V_win,
                                                stream);
  if (st != DAR_OK) return st;
  // rotary keys of every position, like the latent rows
  return hip_status(launch_latent_cast(KR, B, N, d_R, cap, 0, KR_cache, stream));
}

dar_status dar_attn_decode_drope(const void* qC, const void* qR, const void* K_win,
                                 const void* V_win, const void* KR, const void* h_D,
                                 const void* W_upK, const void* W_upV, int B, int ctx_len, int cap,
                                 int heads, int d_k, int d_R, int d_down, int w, dar_dtype dtype,
                                 void* o, void* workspace, size_t* workspace_bytes,
                                 hipStream_t stream) {
  if (!dtype_ok(dtype) || workspace_bytes == nullptr) return DAR_ERR_INVALID_ARG;
  if (B < 1 || ctx_len < 1 || cap < 1 || heads < 1 || d_k < 2 || (d_k & 1) || d_R < 0 ||
      (d_R & 1) || d_down < 1 || w < 0)
    return DAR_ERR_INVALID_ARG;
  if (ctx_len > cap) return DAR_ERR_INVALID_ARG;  // rotary keys of every position <= p are read
  const void* need[] = {qC, qR, KR, h_D, W_upK, W_upV, o};
  for (const void* ptr : need)
    if (!aligned16(ptr)) return DAR_ERR_INVALID_ARG;
  if (w > 0 && (!aligned16(K_win) || !aligned16(V_win))) return DAR_ERR_INVALID_ARG;
  const size_t hd = (size_t)heads * d_k, es = elem_size(dtype);
  const Span ins[8] = {{qC, es * B * hd},
                       {qR, es * B * (size_t)heads * d_R},
                       {K_win, w > 0 ? es * B * hd * (size_t)w : 0},
                       {V_win, w > 0 ? es * B * hd * (size_t)w : 0},
                       {KR, es * B * (size_t)cap * d_R},
                       {h_D, es * B * (size_t)cap * d_down},
                       {W_upK, es * d_down * hd},
                       {W_upV, es * d_down * hd}};
  const Span outs[1] = {{o, es * B * hd}};
  if (!disjoint(outs, 1, ins, 8)) return DAR_ERR_INVALID_ARG;
  if (dtype != DAR_BF16) return DAR_ERR_UNSUPPORTED;
  if (!drope_decode_supported(d_k, d_R, d_down)) return DAR_ERR_UNSUPPORTED;
  if ((size_t)cap * d_down * 2 > 0x7fffffffu) return DAR_ERR_UNSUPPORTED;  // 32-bit offsets
  DropeDecodeProblem p{};
  p.qC = qC;
  p.qR = qR;
  p.K_win = K_win;
  p.V_win = V_win;
  p.KR = KR;
  p.h_D = h_D;
  p.W_upK = W_upK;
  p.W_upV = W_upV;
  p.o = o;
  p.B = B;
  p.ctx = ctx_len;
  p.cap = cap;
  p.H = heads;
  p.d_k = d_k;
  p.d_R = d_R;
  p.d_down = d_down;
  p.w = w;
  const size_t need_bytes = drope_decode_workspace_bytes(p);
  if (workspace == nullptr) {
    *workspace_bytes = need_bytes;
    return DAR_OK;
  }
  if (((uintptr_t)workspace & 255u) != 0) return DAR_ERR_INVALID_ARG;
  if (*workspace_bytes < need_bytes) return DAR_ERR_WORKSPACE;
  {
    const Span ws{workspace, need_bytes};
    for (const Span& x : ins)
      if (overlap(ws, x)) return DAR_ERR_INVALID_ARG;
    if (overlap(ws, outs[0])) return DAR_ERR_INVALID_ARG;
  }
  p.ws = workspace;
  return hip_status(launch_attn_decode_drope(p, stream));
}

// Allocation-free decode: the workspace of dar_attn_decode (RoPE tables and
// per-chunk partials) lives in a file-scope device array, one per GPU, held
// until the process ends.  The host never passes the array's name to a
// kernel: its device address is looked up once per device with
// hipGetSymbolAddress and kept here.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array.
static hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return hipSuccess;
}

dar_status dar_attn_decode_noalloc(const void* q, const void* K_win, const void* V_win,
                                   const void* h_D, const void* W_upK, const void* W_upV, int B,
                                   int ctx_len, int cap, int heads, int d_k, int d_down, int w,
                                   float rope_base, dar_dtype dtype, void* o,
                                   hipStream_t stream) {
  // validation and the workspace size, without touching the device
  size_t need = 0;
  dar_status st = attn_decode_impl(q, K_win, V_win, h_D, W_upK, W_upV, B, ctx_len, nullptr, cap,
                                   heads, d_k, d_down, w, rope_base, dtype, o, nullptr, &need,
                                   stream);
  if (st != DAR_OK) return st;
  if (need > kNoAllocScratchBytes) return DAR_ERR_WORKSPACE;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess) return DAR_ERR_HIP;
  size_t have = kNoAllocScratchBytes;
  return attn_decode_impl(q, K_win, V_win, h_D, W_upK, W_upV, B, ctx_len, nullptr, cap, heads,
                          d_k, d_down, w, rope_base, dtype, o, ws, &have, stream);
}

dar_status dar_attn_decode_varlen(const void* q, const void* K_win, const void* V_win,
                                  const void* h_D, const void* W_upK, const void* W_upV, int B,
                                  const int* ctx_lens, int max_ctx, int cap, int heads, int d_k,
                                  int d_down, int w, float rope_base, dar_dtype dtype, void* o,
                                  void* workspace, size_t* workspace_bytes, hipStream_t stream) {
  if (ctx_lens == nullptr) return DAR_ERR_INVALID_ARG;
  return attn_decode_impl(q, K_win, V_win, h_D, W_upK, W_upV, B, max_ctx, ctx_lens, cap, heads,
                          d_k, d_down, w, rope_base, dtype, o, workspace, workspace_bytes, stream);
}

}  // extern "C"
