// bi_attn.hip — kernels and C ABI of the batch-invariant paged attention library (gfx950).
//
// Kernels
//   page_update_kernel   scatter a step's new K/V rows into their pages (before attention)
//   decode_split_kernel  one wave per (sequence, KV head, split): split partial -> workspace
//   combine_kernel       one wave per (token, q head): ascending fold of the partials, A / L
//   prefill_kernel       one workgroup per (sequence, KV head, query tile): every split of
//                        every row in registers, folded in the loop, A / L in the epilogue
// Both attention routes call subtile_step() and fold_scalars()/fold_elem() from core.hpp on
// byte-identical operand registers, which is what makes their outputs bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "../../include/bi_attn.h"
#include "core.hpp"

#pragma clang fp contract(off)

namespace bi {

constexpr int kWaves = 4;             // waves per workgroup in every attention kernel
constexpr int kThreads = 64 * kWaves;

struct AttnParams {
  const char* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  const int32_t* q_starts;   // prefill only
  float* out;
  float* ws_acc;             // decode: [rows][jmax][D]
  float2* ws_ml;             // decode: [rows][jmax]  (m, l)
  int32_t max_pages, num_pages, batch, total_tokens, max_q_len, max_seq_len;
  int32_t hq, hkv, group, split, policy, num_cus, jmax;
  float cscale;              // softmax scale * log2(e)
};

// Split length of one sequence. Fixed policy: the configured S for every sequence and every
// batch. By-batch policy (comparison only): derived from the batch size and the length.
__device__ __forceinline__ int split_len(const AttnParams& a, int len) {
  if (a.policy == BI_SPLIT_FIXED) return a.split;
  const int by_batch = (2 * a.num_cus + a.batch * a.hkv - 1) / (a.batch * a.hkv);
  const int max_n = (len + 31) / 32;
  const int n = max(1, min(by_batch, max_n));
  const int s = (len + n - 1) / n;
  return max(32, (s + 31) / 32 * 32);
}

// Physical page of logical page `lp` of sequence b, or -1 when it must not be read.
__device__ __forceinline__ int page_of(const AttnParams& a, int b, int lp, int seq_len) {
  if (lp < 0 || lp >= a.max_pages || lp * kPage >= seq_len) return -1;
  const int p = a.page_table[(size_t)b * a.max_pages + lp];
  return (p >= 0 && p < a.num_pages) ? p : -1;
}

template <typename E, int D>
__device__ __forceinline__ const char* kv_row(const char* cache, const AttnParams& a, int page,
                                              int kvh, int slot) {
  return cache + (((size_t)page * a.hkv + kvh) * kPage + slot) * (size_t)(D * sizeof(E));
}

// ------------------------------------------------------------------------------------------
// Decode: one wave per split. Operands stream from HBM straight into MFMA registers.
template <typename E, int D, int NB>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(AttnParams a) {
  using F = Frag<E, D>;
  constexpr int NM = D / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int j = blockIdx.x * kWaves + wave;
  const int seq_len = a.seq_lens[b];
  if (seq_len <= 0 || seq_len > a.max_seq_len) return;   // combine writes NaN for the row
  const int pos = seq_len - 1;
  const int S = split_len(a, seq_len);
  const int k_begin = j * S;
  if (k_begin > pos || j >= a.jmax) return;
  const int k_end = min(k_begin + S, pos + 1);

  typename F::Q qf[NB];
  RowState<D> st[NB];
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int hl = cb * 16 + c;   // head within the group
    if (hl < a.group) {
      const char* row = a.q + ((size_t)b * a.hq + kvh * a.group + hl) * (size_t)(D * sizeof(E));
      F::load_q(qf[cb], row, g);
    } else {
      F::zero_q(qf[cb]);
    }
  }
  for (int key0 = k_begin; key0 < k_end; key0 += kSubTile) {
    typename F::K kf;
    typename F::VRaw vr;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int page = page_of(a, b, (key0 >> 4) + kb, seq_len);
      if (page >= 0) F::load_k_block(kf, kb, kv_row<E, D>(a.k_cache, a, page, kvh, c), g);
      else F::zero_k_block(kf, kb);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = key0 + F::vkey(i, g);
      const int page = page_of(a, b, key >> 4, seq_len);
      if (page >= 0 && key < seq_len) F::load_v_key(vr, i, kv_row<E, D>(a.v_cache, a, page, kvh, key & 15), c);
      else F::zero_v_key(vr, i);
    }
    typename F::V vf;
    F::pack_v(vf, vr);
    const bool first = key0 == k_begin;
    const bool mask = key0 + kSubTile - 1 > pos;
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
      subtile_step<E, D>(st[cb], qf[cb], kf, vf, a.cscale, key0, g, pos, true, first, mask, false);
  }
  // Partial of split j for every real head of the block.
#pragma unroll
  for (int cb = 0; cb < NB; ++cb) {
    const int hl = cb * 16 + c;
    if (hl >= a.group) continue;
    const size_t row = (size_t)b * a.hq + kvh * a.group + hl;
    const size_t pidx = row * a.jmax + j;
    float* dst = a.ws_acc + pidx * D + 4 * g * NM;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int mb = 0; mb < NM; mb += 4) {
        f32x4 v = {st[cb].acc[mb][r], st[cb].acc[mb + 1][r], st[cb].acc[mb + 2][r], st[cb].acc[mb + 3][r]};
        *(f32x4*)(dst + r * NM + mb) = v;
      }
    if (g == 0) a.ws_ml[pidx] = make_float2(st[cb].m, st[cb].l);
  }
}

// Combine: one wave per (token, q head); lane t owns dims t * D/64 ... in ascending j.
template <int D>
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnParams a) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= (size_t)a.batch * a.hq) return;
  const int b = (int)(row / a.hq);
  const int seq_len = a.seq_lens[b];
  float* o = a.out + row * D + lane * PER;
  if (seq_len <= 0 || seq_len > a.max_seq_len) {
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = __builtin_nanf("");
    return;
  }
  const int S = split_len(a, seq_len);
  const int J = (seq_len - 1) / S + 1;
  const float2* ml = a.ws_ml + row * a.jmax;
  const float* acc = a.ws_acc + row * a.jmax * D + lane * PER;
  float M = 0.f, L = 0.f, A[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) A[e] = 0.f;
  constexpr int U = 8;
  for (int j0 = 0; j0 < J; j0 += U) {
    float2 mlj[U];
    float accj[U][PER];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < J) {
        mlj[u] = ml[j0 + u];
#pragma unroll
        for (int e = 0; e < PER; ++e) accj[u][e] = acc[(size_t)(j0 + u) * D + e];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < J) {
        const bool first = (j0 + u) == 0;
        float fa, fb;
        fold_scalars(M, L, mlj[u].x, mlj[u].y, first, fa, fb);
#pragma unroll
        for (int e = 0; e < PER; ++e) A[e] = fold_elem(A[e], accj[u][e], fa, fb, first);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = A[e] / L;
}

// ------------------------------------------------------------------------------------------
// Prefill: a workgroup owns a tile of query columns (token-major: column = token * G + head)
// of one (sequence, KV head) and walks every split that any of its rows needs. K/V sub-tiles
// are staged once in LDS and shared by the four waves; each wave holds NBW column blocks.
template <int D, typename E> struct Lds {
  static constexpr int ROWB = D * (int)sizeof(E);
  static constexpr int STRIDE = ROWB + 16;              // pad rows against bank conflicts
  static constexpr int BYTES = 2 * kSubTile * STRIDE;   // K then V
};

template <typename E, int D, int NBW>
__global__ __launch_bounds__(kThreads) void prefill_kernel(AttnParams a) {
  using F = Frag<E, D>;
  using LD = Lds<D, E>;
  constexpr int NM = D / 16;
  constexpr int COLS = kWaves * NBW * 16;
  __shared__ __attribute__((aligned(16))) char lds[LD::BYTES];
  char* lds_k = lds;
  char* lds_v = lds + kSubTile * LD::STRIDE;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int b = blockIdx.z, kvh = blockIdx.y;
  const int G = a.group;
  const int tq = COLS / G;                       // tokens per tile (G divides COLS)
  const int q0 = a.q_starts[b], q1 = a.q_starts[b + 1];
  const int n_new = q1 - q0;
  const int t0 = blockIdx.x * tq;
  if (t0 >= n_new || q1 > a.total_tokens || q0 < 0) return;
  const int seq_len = a.seq_lens[b];
  const bool bad_seq = seq_len > a.max_seq_len || n_new > seq_len;
  const int first_pos = seq_len - n_new;
  const int t_last = min(t0 + tq, n_new) - 1;
  const int pos_max_wg = first_pos + t_last;
  const int S = split_len(a, seq_len);

  typename F::Q qf[NBW];
  RowState<D> st[NBW];
  float Mrow[NBW], Lrow[NBW];
  f32x4 Arow[NBW][NM];
  int pos_c[NBW], blk_min[NBW], blk_max[NBW];
  bool valid_c[NBW];
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int col0 = (wave * NBW + cb) * 16;
    const int col = col0 + c;
    const int tok = t0 + col / G;
    valid_c[cb] = tok < n_new && !bad_seq;
    pos_c[cb] = valid_c[cb] ? first_pos + tok : -1;
    // block-wide position range of valid columns (wave-uniform)
    const int tok_lo = t0 + col0 / G, tok_hi = min(t0 + (col0 + 15) / G, n_new - 1);
    blk_min[cb] = (tok_lo < n_new && !bad_seq) ? first_pos + tok_lo : 0x7fffffff;
    blk_max[cb] = (tok_lo < n_new && !bad_seq) ? first_pos + tok_hi : -1;
    if (valid_c[cb]) {
      const char* row = a.q + ((size_t)(q0 + tok) * a.hq + kvh * G + col % G) * (size_t)(D * sizeof(E));
      F::load_q(qf[cb], row, g);
    } else {
      F::zero_q(qf[cb]);
    }
    Mrow[cb] = 0.f;
    Lrow[cb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) Arow[cb][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int wave_max = -1;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) wave_max = max(wave_max, blk_max[cb]);

  const int n_splits = bad_seq ? 0 : pos_max_wg / S + 1;
  for (int j = 0; j < n_splits; ++j) {
    const int k_begin = j * S;
    const int k_end = min(k_begin + S, pos_max_wg + 1);
    for (int key0 = k_begin; key0 < k_end; key0 += kSubTile) {
      __syncthreads();
      // Stage K and V rows [key0, key0 + 32) in LDS; V rows at or past seq_len and rows of
      // absent pages are zero, so no stale cache bytes reach an MFMA.
      constexpr int CHUNKS = LD::ROWB / 16;               // 16-byte chunks per row
      constexpr int TOTAL = 2 * kSubTile * CHUNKS;
      for (int idx = threadIdx.x; idx < TOTAL; idx += kThreads) {
        const int which = idx / (kSubTile * CHUNKS);       // 0 = K, 1 = V
        const int rem = idx - which * kSubTile * CHUNKS;
        const int r = rem / CHUNKS, ch = rem - r * CHUNKS;
        const int key = key0 + r;
        const int page = page_of(a, b, key >> 4, seq_len);
        u32x4 val = {0, 0, 0, 0};
        if (page >= 0 && (which == 0 || key < seq_len)) {
          const char* src = kv_row<E, D>(which ? a.v_cache : a.k_cache, a, page, kvh, key & 15);
          val = *(const u32x4*)(src + ch * 16);
        }
        *(u32x4*)((which ? lds_v : lds_k) + r * LD::STRIDE + ch * 16) = val;
      }
      __syncthreads();
      if (wave_max < key0) continue;                      // no row of this wave sees these keys
      typename F::K kf;
      typename F::VRaw vr;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) F::load_k_block(kf, kb, lds_k + (16 * kb + c) * LD::STRIDE, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) F::load_v_key(vr, i, lds_v + F::vkey(i, g) * LD::STRIDE, c);
      typename F::V vf;
      F::pack_v(vf, vr);
      const bool first = key0 == k_begin;
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb) {
        if (blk_max[cb] < key0) continue;                 // whole block past its rows
        // mask: some key lies past some valid row; partial: some valid row has not reached
        // key0 and must keep its state (only when a block holds several tokens, G < 16).
        const bool mask = key0 + kSubTile - 1 > blk_min[cb];
        const bool partial = key0 > blk_min[cb];
        subtile_step<E, D>(st[cb], qf[cb], kf, vf, a.cscale, key0, g, pos_c[cb],
                           pos_c[cb] >= key0, first, mask, partial);
      }
    }
    // Fold split j into every row whose position reaches it.
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      if (blk_max[cb] < k_begin) continue;
      const bool act = pos_c[cb] >= k_begin;
      float M = Mrow[cb], L = Lrow[cb], fa, fb;
      fold_scalars(M, L, st[cb].m, st[cb].l, j == 0, fa, fb);
      if (act) {
        Mrow[cb] = M;
        Lrow[cb] = L;
#pragma unroll
        for (int mb = 0; mb < NM; ++mb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            Arow[cb][mb][r] = fold_elem(Arow[cb][mb][r], st[cb].acc[mb][r], fa, fb, j == 0);
      }
    }
  }
  // Epilogue: out = A / L for every valid row.
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int col = (wave * NBW + cb) * 16 + c;
    const int tok = t0 + col / G;
    if (tok >= n_new) continue;
    float* dst = a.out + ((size_t)(q0 + tok) * a.hq + kvh * G + col % G) * D + 4 * g * NM;
    const bool ok = valid_c[cb];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int mb = 0; mb < NM; mb += 4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ok ? Arow[cb][mb + e][r] / Lrow[cb] : __builtin_nanf("");
        *(f32x4*)(dst + r * NM + mb) = v;
      }
  }
}

// ------------------------------------------------------------------------------------------
// Page update: one thread per 16-byte chunk of a (token, KV head) row of K or V.
template <int ROWB>
__global__ __launch_bounds__(256) void page_update_kernel(const char* k_new, const char* v_new,
                                                          const int32_t* q_starts,
                                                          const int32_t* seq_lens,
                                                          const int32_t* page_table,
                                                          int max_pages, int num_pages, int batch,
                                                          int total_tokens, int hkv,
                                                          char* k_cache, char* v_cache) {
  constexpr int CH = ROWB / 16;
  const size_t n = (size_t)total_tokens * hkv * CH * 2;
  for (size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (size_t)gridDim.x * blockDim.x) {
    const int which = (int)(idx % 2);
    const size_t rest = idx / 2;
    const int ch = (int)(rest % CH);
    const size_t th = rest / CH;
    const int h = (int)(th % hkv);
    const int t = (int)(th / hkv);
    // sequence of token t: last b with q_starts[b] <= t
    int lo = 0, hi = batch;                       // invariant: q_starts[lo] <= t < q_starts[hi]
    if (t < q_starts[0] || t >= q_starts[batch]) continue;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (q_starts[mid] <= t) lo = mid; else hi = mid;
    }
    const int bq = lo;
    const int n_new = q_starts[bq + 1] - q_starts[bq];
    const int pos = seq_lens[bq] - n_new + (t - q_starts[bq]);
    if (pos < 0) continue;
    const int lp = pos / kPage;
    if (lp >= max_pages) continue;
    const int page = page_table[(size_t)bq * max_pages + lp];
    if (page < 0 || page >= num_pages) continue;
    const size_t src = ((size_t)t * hkv + h) * ROWB + ch * 16;
    const size_t dst = (((size_t)page * hkv + h) * kPage + (pos % kPage)) * ROWB + ch * 16;
    if (which == 0) *(u32x4*)(k_cache + dst) = *(const u32x4*)(k_new + src);
    else *(u32x4*)(v_cache + dst) = *(const u32x4*)(v_new + src);
  }
}

}  // namespace bi

// ==========================================================================================
// C ABI (declared and documented in include/bi_attn.h)
// ==========================================================================================
namespace {

using namespace bi;

int g_cu_count[64];   // per device; 0 = not queried yet (benign race: same value)

int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && g_cu_count[dev] > 0) return g_cu_count[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) g_cu_count[dev] = n;
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_cfg(const bi_attn_cfg* c) {
  if (!c) return BI_EINVAL;
  if (c->num_q_heads <= 0 || c->num_kv_heads <= 0 || c->num_q_heads % c->num_kv_heads) return BI_EINVAL;
  if (c->dtype != BI_F32 && c->dtype != BI_BF16) return BI_EINVAL;
  if (c->split_policy != BI_SPLIT_FIXED && c->split_policy != BI_SPLIT_BY_BATCH) return BI_EINVAL;
  if (!(c->softmax_scale >= 0.f) || c->softmax_scale == __builtin_inff()) return BI_EINVAL;
  if (c->split_size <= 0 || c->page_size <= 0 || c->head_dim <= 0) return BI_EINVAL;
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G > 64 || (G & (G - 1))) return BI_EUNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return BI_EUNSUPPORTED;
  if (c->page_size != kPage) return BI_EUNSUPPORTED;
  if (c->split_size % kSubTile) return BI_EUNSUPPORTED;
  return BI_OK;
}

float cscale_of(const bi_attn_cfg* c) {
  const double s = c->softmax_scale > 0.f ? (double)c->softmax_scale : 1.0 / sqrt((double)c->head_dim);
  return (float)(s * 1.4426950408889634074);   // log2(e)
}

int64_t jmax_of(const bi_attn_cfg* c, int64_t batch, int64_t max_seq_len) {
  if (max_seq_len <= 0) return 1;
  if (c->split_policy == BI_SPLIT_FIXED) return (max_seq_len + c->split_size - 1) / c->split_size;
  // by-batch: at most ceil(2 CUs / (batch Hkv)) splits, and never more than ceil(len / 32)
  const int64_t b = batch > 0 ? batch : 1;
  const int64_t by_batch = (2 * (int64_t)cu_count() + b * c->num_kv_heads - 1) / (b * c->num_kv_heads);
  const int64_t by_len = (max_seq_len + 31) / 32;
  return by_batch < by_len ? (by_batch > 0 ? by_batch : 1) : by_len;
}

size_t ws_ml_bytes(int64_t rows, int64_t jmax) { return (size_t)((rows * jmax * 8 + 255) / 256 * 256); }

size_t ws_bytes(const bi_attn_cfg* c, int64_t tokens, int64_t batch_for_policy, int64_t max_seq_len) {
  const int64_t rows = tokens * c->num_q_heads;
  const int64_t jmax = jmax_of(c, batch_for_policy, max_seq_len);
  return ws_ml_bytes(rows, jmax) + (size_t)(rows * jmax * c->head_dim * 4);
}

AttnParams base_params(const bi_attn_cfg* c) {
  AttnParams a{};
  a.hq = c->num_q_heads;
  a.hkv = c->num_kv_heads;
  a.group = c->num_q_heads / c->num_kv_heads;
  a.split = c->split_size;
  a.policy = c->split_policy;
  a.cscale = cscale_of(c);
  a.num_cus = c->split_policy == BI_SPLIT_BY_BATCH ? cu_count() : 0;
  return a;
}

int launched() { return hipGetLastError() == hipSuccess ? BI_OK : BI_EHIP; }

template <typename E, int D>
int launch_decode(const AttnParams& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.jmax + kWaves - 1) / kWaves), (unsigned)a.hkv, (unsigned)a.batch);
  if (a.group <= 16) hipLaunchKernelGGL((decode_split_kernel<E, D, 1>), grid, dim3(kThreads), 0, s, a);
  else if (a.group == 32) hipLaunchKernelGGL((decode_split_kernel<E, D, 2>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((decode_split_kernel<E, D, 4>), grid, dim3(kThreads), 0, s, a);
  if (launched() != BI_OK) return BI_EHIP;
  const unsigned rows = (unsigned)((int64_t)a.batch * a.hq);
  hipLaunchKernelGGL((combine_kernel<D>), dim3((rows + kWaves - 1) / kWaves), dim3(kThreads), 0, s, a);
  return launched();
}

constexpr int kPrefillNBW = 2;

template <typename E, int D>
int launch_prefill(const AttnParams& a, hipStream_t s) {
  const int cols = kWaves * kPrefillNBW * 16;
  const int tq = cols / a.group;
  const dim3 grid((unsigned)((a.max_q_len + tq - 1) / tq), (unsigned)a.hkv, (unsigned)a.batch);
  hipLaunchKernelGGL((prefill_kernel<E, D, kPrefillNBW>), grid, dim3(kThreads), 0, s, a);
  return launched();
}

}  // namespace

extern "C" {

const char* bi_status_string(int status) {
  switch (status) {
    case BI_OK: return "ok";
    case BI_EINVAL: return "invalid argument";
    case BI_EUNSUPPORTED: return "unsupported configuration";
    case BI_EWORKSPACE: return "workspace missing or too small";
    case BI_EHIP: return "HIP runtime error at launch";
    default: return "unknown status";
  }
}

size_t bi_attn_workspace_bytes(const bi_attn_cfg* cfg, int32_t rows_tokens, int32_t max_seq_len) {
  if (check_cfg(cfg) != BI_OK || rows_tokens < 0 || max_seq_len < 0) return 0;
  // batch-free bound for the by-batch policy: the split count is largest at batch 1
  return ws_bytes(cfg, rows_tokens, 1, max_seq_len);
}

int bi_kv_page_update(const bi_attn_cfg* cfg, const void* k_new, const void* v_new,
                      const int32_t* q_starts, const int32_t* seq_lens, const int32_t* page_table,
                      int32_t max_pages, int32_t num_pages, int32_t batch, int32_t total_tokens,
                      void* k_cache, void* v_cache, hipStream_t stream) {
  int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || total_tokens < 0 || max_pages < 0 || num_pages < 0) return BI_EINVAL;
  if (batch == 0 || total_tokens == 0) return BI_OK;
  if (!k_new || !v_new || !q_starts || !seq_lens || !page_table || !k_cache || !v_cache) return BI_EINVAL;
  if (max_pages == 0 || num_pages == 0) return BI_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache)) return BI_EINVAL;
  const int rowb = cfg->head_dim * (cfg->dtype == BI_BF16 ? 2 : 4);
  const size_t work = (size_t)total_tokens * cfg->num_kv_heads * (rowb / 16) * 2;
  const unsigned blocks = (unsigned)((work + 255) / 256 < 65536 ? (work + 255) / 256 : 65536);
#define BI_PU(RB)                                                                                 \
  hipLaunchKernelGGL((page_update_kernel<RB>), dim3(blocks), dim3(256), 0, stream,               \
                     (const char*)k_new, (const char*)v_new, q_starts, seq_lens, page_table,      \
                     max_pages, num_pages, batch, total_tokens, cfg->num_kv_heads, (char*)k_cache, \
                     (char*)v_cache)
  if (rowb == 128) BI_PU(128);
  else if (rowb == 256) BI_PU(256);
  else BI_PU(512);
#undef BI_PU
  return launched();
}

int bi_attn_decode(const bi_attn_cfg* cfg, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || max_seq_len < 0 || max_pages < 0 || num_pages < 0) return BI_EINVAL;
  if (batch == 0) return BI_OK;
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out) return BI_EINVAL;
  if (max_seq_len == 0 || max_pages == 0 || num_pages == 0) return BI_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return BI_EINVAL;
  const size_t need = ws_bytes(cfg, batch, batch, max_seq_len);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return BI_EWORKSPACE;
  AttnParams a = base_params(cfg);
  a.q = (const char*)q;
  a.k_cache = (const char*)k_cache;
  a.v_cache = (const char*)v_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.batch = batch;
  a.total_tokens = batch;
  a.max_q_len = 1;
  a.max_seq_len = max_seq_len;
  a.jmax = (int32_t)jmax_of(cfg, batch, max_seq_len);
  a.ws_ml = (float2*)workspace;
  a.ws_acc = (float*)((char*)workspace + ws_ml_bytes((int64_t)batch * cfg->num_q_heads, a.jmax));
  const bool bf = cfg->dtype == BI_BF16;
  if (cfg->head_dim == 128) return bf ? launch_decode<__bf16, 128>(a, stream) : launch_decode<float, 128>(a, stream);
  return bf ? launch_decode<__bf16, 64>(a, stream) : launch_decode<float, 64>(a, stream);
}

int bi_attn_prefill(const bi_attn_cfg* cfg, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                    const int32_t* q_starts, const int32_t* seq_lens, int32_t batch,
                    int32_t total_tokens, int32_t max_q_len, int32_t max_seq_len, float* out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || total_tokens < 0 || max_q_len < 0 || max_seq_len < 0 || max_pages < 0 || num_pages < 0)
    return BI_EINVAL;
  if (batch == 0 || total_tokens == 0 || max_q_len == 0) return BI_OK;
  if (!q || !k_cache || !v_cache || !page_table || !q_starts || !seq_lens || !out) return BI_EINVAL;
  if (max_seq_len == 0 || max_pages == 0 || num_pages == 0) return BI_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return BI_EINVAL;
  AttnParams a = base_params(cfg);
  a.q = (const char*)q;
  a.k_cache = (const char*)k_cache;
  a.v_cache = (const char*)v_cache;
  a.page_table = page_table;
  a.seq_lens = seq_lens;
  a.q_starts = q_starts;
  a.out = out;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  a.batch = batch;
  a.total_tokens = total_tokens;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  const bool bf = cfg->dtype == BI_BF16;
  if (cfg->head_dim == 128) return bf ? launch_prefill<__bf16, 128>(a, stream) : launch_prefill<float, 128>(a, stream);
  return bf ? launch_prefill<__bf16, 64>(a, stream) : launch_prefill<float, 64>(a, stream);
}

}  // extern "C"
