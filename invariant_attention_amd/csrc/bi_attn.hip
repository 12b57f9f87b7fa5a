// bi_attn.hip — kernels and C ABI of the batch-invariant paged attention library (gfx950).
//
// Kernels
//   page_update_kernel   scatter a step's new K/V rows into their pages (before attention)
//   decode_split_kernel  one wave per (sequence, KV head, split): split partial -> workspace;
//                        its APPEND form also writes each sequence's new token into its page
//   combine_kernel       rows of at most 32 splits: one wave per 256 floats of a (token, KV
//                        head)'s partials; ascending fold of the partials, A / L
//   combine_rows_kernel  rows of more than 32 splits: one workgroup per (token, q head) row,
//                        the row's reference, L and element chains in separate waves
//   prefill_kernel       one workgroup per (sequence, KV head, query tile): every split of
//                        every row in registers, folded in the loop, A / L in the epilogue
// Both attention routes call subtile_step() and fold_scalars()/fold_elem() from core.hpp on
// byte-identical operand registers, which is what makes their outputs bit-identical.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include <algorithm>

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
  const int32_t* k_starts;   // dense (varlen) prefill only: first K/V row of each sequence
  const char* k_new;         // decode with append: the new token of sequence b, [batch][Hkv][D]
  const char* v_new;
  float* out;
  float* ws_acc;             // decode: [batch Hkv][jmax][group][D]
  float2* ws_ml;             // decode: [batch Hkv][jmax][group]  (m, l)
  int32_t max_pages, num_pages, batch, total_tokens, max_q_len, max_seq_len;
  int32_t k_rows;            // dense: rows of the K and V arrays
  int32_t hq, hkv, group, split, policy, num_cus, jmax;
  float cscale;              // softmax scale * log2(e)
};

// Split length of one sequence. Fixed policy: the configured S for every sequence and every
// batch. By-batch policies (comparison only): derived from the batch size and the length,
// with a split count of about 2 per CU (BI_SPLIT_BY_BATCH) or 8 per CU, the waves the
// attention kernels keep resident (BI_SPLIT_BY_BATCH_FILL), over the batch's KV heads.
__device__ __forceinline__ int split_len(const AttnParams& a, int len) {
  if (a.policy == BI_SPLIT_FIXED) return a.split;
  const int per_cu = a.policy == BI_SPLIT_BY_BATCH_FILL ? 8 : 2;
  const int by_batch = (per_cu * a.num_cus + a.batch * a.hkv - 1) / (a.batch * a.hkv);
  const int max_n = (len + 31) / 32;
  const int n = max(1, min(by_batch, max_n));
  const int s = (len + n - 1) / n;
  return max(32, (s + 31) / 32 * 32);
}

// Index of the partial of split j of query row `row` (= b Hq + h) in the workspace: the rows of
// one (sequence, KV head) are adjacent for each split, so one split's partials are contiguous.
__device__ __forceinline__ size_t part_index(const AttnParams& a, size_t row, int j) {
  return (row / a.group * a.jmax + j) * a.group + row % a.group;
}

// Physical page of logical page `lp` of sequence b, or -1 when it must not be read.
__device__ __forceinline__ int page_of(const AttnParams& a, int b, int lp, int seq_len) {
  if (lp < 0 || lp >= a.max_pages || lp * kPage >= seq_len) return -1;
  const int p = a.page_table[(size_t)b * a.max_pages + lp];
  return (p >= 0 && p < a.num_pages) ? p : -1;
}
// The same without a branch around the load (an out-of-range lp reads entry 0 of row b,
// which exists, and discards it), for code that keeps other loads in flight meanwhile.
__device__ __forceinline__ int page_of_nb(const AttnParams& a, int b, int lp, int seq_len) {
  const bool ok = lp >= 0 && lp < a.max_pages && lp * kPage < seq_len;
  const int p = a.page_table[(size_t)b * a.max_pages + (ok ? lp : 0)];
  return (ok && p >= 0 && p < a.num_pages) ? p : -1;
}

// Entry i of a read-only int array through the scalar data cache (i made wave-uniform): the
// load waits on the scalar counter only, so the vector loads in flight are not waited for.
__device__ __forceinline__ int scalar_load_i32(const int32_t* p, int i) {
  const __attribute__((address_space(4))) int32_t* cp = (const __attribute__((address_space(4))) int32_t*)p;
  return cp[__builtin_amdgcn_readfirstlane(i)];
}

// Rows read in place of a page that must not be dereferenced (table entry absent, outside the
// pool, or past the sequence end). K rows are NaN, so a query row whose causal window needs the
// page comes out NaN while masked keys ignore them; V rows are zero, so a zero probability
// times V stays zero. Sized for the widest row (fp32, D 128). Loads are then unconditional.
constexpr int kMaxRowBytes = 512;
struct NanRows {
  uint32_t w[kPage * kMaxRowBytes / 4];
  constexpr NanRows() : w() {
    for (int i = 0; i < kPage * kMaxRowBytes / 4; ++i) w[i] = 0x7fc07fc0u;   // bf16 and fp32 NaN
  }
};
// (global, not constant, address space: a pointer that selects between them and a cache page
// stays a global pointer, so its loads are global loads)
__device__ __attribute__((aligned(256))) NanRows kNanRows;
__device__ __attribute__((aligned(256))) uint32_t kZeroRows[kPage * kMaxRowBytes / 4];

template <typename E, int D>
__device__ __forceinline__ const char* kv_row(const char* cache, const AttnParams& a, int page,
                                              int kvh, int slot) {
  return cache + (((size_t)page * a.hkv + kvh) * kPage + slot) * (size_t)(D * sizeof(E));
}

// ------------------------------------------------------------------------------------------
// Decode. The work items are the splits (b, j) of every sequence, for every KV head (every
// split but the last first, then the last splits). The grid holds as many workgroups as the
// device keeps resident; each owns an equal strided share of the items (so every CU gets the
// same share, within one item), and its waves take the share's items one at a time as they
// finish the previous one. Per item, operands stream from HBM straight into MFMA registers with
// two sub-tiles in flight: the loads of sub-tile t+1 are issued before sub-tile t is computed.
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Waves per decode workgroup: 8 (two per SIMD, one workgroup per CU) for the bf16 kernel with one
// column block, whose 256 VGPRs allow two waves per SIMD; else 4 (one per SIMD).
template <typename E, int NB> struct DecWaves {
  static constexpr int value = (sizeof(E) == 2 && NB == 1) ? 8 : 4;
};

template <typename E, int D, int NB, bool APPEND>
__global__ __launch_bounds__((64 * DecWaves<E, NB>::value), 1) void decode_split_kernel(AttnParams a) {
  using F = Frag<E, D>;
  constexpr int NWV = DecWaves<E, NB>::value;
  using KOp = typename F::KOp;
  using VRow = typename F::VRow;
  constexpr int NKS = F::NKS;
  constexpr int NM = D / 16;
  constexpr int ROWB = F::ROWB;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  // Work items are the pairs I = i Hkv + h of split item i (below) and KV head h. Workgroup k
  // owns I = k, k + G, k + 2G, ... (G workgroups), and its waves take the next of those from a
  // counter in LDS whenever they need one: the two waves that share a SIMD do not progress at
  // the same rate (with a fixed share per wave, the second wave of each SIMD finished about
  // 1.35x later than the first), so a fixed share would leave the faster ones idle at the end.
  // Which wave computes a split does not change its bits.
  __shared__ int lds_next;
  // per wave: one split's accumulators [NB 16 rows][D], staged for contiguous stores (only
  // this wave touches its slice, and one wave's LDS accesses complete in order)
  __shared__ __attribute__((aligned(16))) float lds_part_all[NWV][NB * 16 * D];
  float* lds_part = lds_part_all[__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6))];
  // the first 64 sequence lengths, for the last-split lookup of a batch of up to 64 (LDS reads
  // wait on their own counter, so that lookup never waits for the K/V loads in flight)
  __shared__ int lds_len[64];
  if (threadIdx.x < 64) lds_len[threadIdx.x] = (int)threadIdx.x < a.batch ? a.seq_lens[threadIdx.x] : 0;
  if (threadIdx.x == 0) lds_next = 0;
  __syncthreads();
  auto claim = [&]() {
    int n = 0;
    if (lane == 0) n = atomicAdd(&lds_next, 1);
    return (int)blockIdx.x + __builtin_amdgcn_readfirstlane(n) * (int)gridDim.x;
  };

  // Sequences are read 64 at a time, one per lane: length and split count (0 when the length
  // is out of range; the combine writes NaN for such a row).
  auto chunk_len = [&](int cb) {
    const int bb = cb + lane;
    return bb < a.batch ? a.seq_lens[bb] : 0;
  };
  auto splits_of = [&](int len) {
    return (len > 0 && len <= a.max_seq_len) ? (len - 1) / split_len(a, len) + 1 : 0;
  };
  // Items in two runs: first every split but the last of each sequence (b, then j), then the
  // last split of each sequence. A last split is the only one that can be short, so the items
  // handed out last (to the waves that get one more) are the cheap ones.
  int total_full = 0, total_last = 0;
  for (int cb = 0; cb < a.batch; cb += 64) {
    const int nj = splits_of(chunk_len(cb));
    total_full += wave_sum_i(max(nj - 1, 0));
    total_last += wave_sum_i(nj > 0 ? 1 : 0);
  }
  total_full = __builtin_amdgcn_readfirstlane(total_full);
  const int total = total_full + __builtin_amdgcn_readfirstlane(total_last);
  const int n_items = total * a.hkv;
  const int I0 = claim();
  if (I0 >= n_items) return;
  // Item i -> (sequence, split, length) for increasing i: one cursor per run over the chunks
  // of 64 sequences (inclusive prefix sums of the run's per-sequence item counts in incl;
  // `before` items of the run precede the chunk).
  auto count_of = [&](int run, int len) {
    const int nj = splits_of(len);
    return run == 0 ? max(nj - 1, 0) : (nj > 0 ? 1 : 0);
  };
  int cb0 = 0, before0 = 0, incl0 = wave_incl_scan(count_of(0, chunk_len(0)), lane);
  int cb1 = 0, before1 = 0, incl1 = wave_incl_scan(count_of(1, chunk_len(0)), lane);
  auto seek = [&](int run, int k, int& cb, int& before, int& incl) {
    for (;;) {
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (before + tot > k) break;
      before += tot;
      cb += 64;
      incl = wave_incl_scan(count_of(run, chunk_len(cb)), lane);
    }
    const int nb = __builtin_popcountll(__builtin_amdgcn_ballot_w64(before + incl <= k));
    return nb;
  };
  // With a fixed split size the last run is ordered by the last split's sub-tile count,
  // largest first (ties by sequence), so the items taken last, at the end of the run, are the
  // cheapest.
  const bool by_cost = a.policy == BI_SPLIT_FIXED;
  const int cmax = (a.split + kSubTile - 1) / kSubTile;
  auto last_cost = [&](int len) {
    const int nj = splits_of(len);
    return nj > 0 ? (len - (nj - 1) * a.split + kSubTile - 1) / kSubTile : 0;
  };
  // sequence of the k-th last split in (cost descending, sequence) order
  auto last_by_cost = [&](int k) {
    if (a.batch <= 64) {   // one chunk, from LDS (lane id behind an empty asm, as below)
      int lid = lane;
      asm volatile("" : "+v"(lid));
      const int cost = last_cost(lds_len[lid]);
      for (int cst = cmax; cst >= 1; --cst) {
        unsigned long long m = __builtin_amdgcn_ballot_w64(cost == cst);
        const int n = __builtin_popcountll(m);
        if (k >= n) {
          k -= n;
          continue;
        }
        for (int t = 0; t < k; ++t) m &= m - 1;   // drop the k lowest set lanes
        return (int)__builtin_ctzll(m);
      }
      return 0;   // not reached: k < total_last
    }
    for (int cst = cmax; cst >= 1; --cst) {
      int cnt = 0;
      for (int cb = 0; cb < a.batch; cb += 64) cnt += wave_sum_i(last_cost(chunk_len(cb)) == cst ? 1 : 0);
      cnt = __builtin_amdgcn_readfirstlane(cnt);
      if (k >= cnt) {
        k -= cnt;
        continue;
      }
      for (int cb = 0;; cb += 64) {
        const unsigned long long m = __builtin_amdgcn_ballot_w64(last_cost(chunk_len(cb)) == cst);
        const int n = __builtin_popcountll(m);
        if (k < n) {
          unsigned long long mm = m;
          for (int t = 0; t < k; ++t) mm &= mm - 1;   // drop the k lowest set lanes
          return cb + (int)__builtin_ctzll(mm);
        }
        k -= n;
      }
    }
    return 0;   // not reached: k < total_last
  };
  auto locate = [&](int i, int& ob, int& oj, int& olen) {
    if (i < total_full) {
      const int nb = seek(0, i, cb0, before0, incl0);
      ob = cb0 + nb;
      oj = i - before0 - (nb > 0 ? __builtin_amdgcn_readlane(incl0, nb - 1) : 0);
      olen = scalar_load_i32(a.seq_lens, ob);
    } else {
      if (by_cost) {
        ob = __builtin_amdgcn_readfirstlane(last_by_cost(i - total_full));
      } else {
        const int nb = seek(1, i - total_full, cb1, before1, incl1);
        ob = cb1 + nb;
      }
      olen = scalar_load_i32(a.seq_lens, ob);
      oj = splits_of(olen) - 1;
    }
  };
  int b = 0, j = 0, len0 = 0;
  locate(I0 / a.hkv, b, j, len0);

  const size_t head_stride = (size_t)kPage * ROWB;
  const size_t page_stride = (size_t)a.hkv * head_stride;
  // Every load below is unconditional: absent pages read kNanRows / kZeroRows and heads past
  // the group read zero q, so no branch separates a buffer's loads from their use, and the
  // loads of the next sub-tile stay in flight while the current one is computed.
  const char* nan_rows = (const char*)&kNanRows;
  const char* zero_rows = (const char*)kZeroRows;

  // A unit is up to 32 sub-tiles of one split (a window of 64 pages, one page id per lane).
  // The loads of a unit's first sub-tile are issued while the previous unit's last sub-tile is
  // computed, so the stream of loads does not stop between splits.
  struct Unit {
    int b, j, kvh, w0, seq_len, k_begin, nsub, nw;
  };
  auto make_unit = [&](int ub, int uj, int ukvh, int w0, int len) {
    Unit u;
    u.b = ub;
    u.j = uj;
    u.kvh = ukvh;
    u.w0 = w0;
    u.seq_len = len;
    const int S = split_len(a, len);
    u.k_begin = uj * S;
    u.nsub = (min(u.k_begin + S, len) - u.k_begin + kSubTile - 1) / kSubTile;
    u.nw = min(32, u.nsub - w0);
    return u;
  };
  // the unit after u: the next window of its split, else window 0 of the wave's next item
  auto next_unit = [&](const Unit& u, Unit& un) {
    if (u.w0 + 32 < u.nsub) {
      un = make_unit(u.b, u.j, u.kvh, u.w0 + 32, u.seq_len);
      return true;
    }
    const int I = claim();
    if (I >= n_items) return false;
    int nb2, nj2, len2;
    locate(I / a.hkv, nb2, nj2, len2);
    un = make_unit(nb2, nj2, I % a.hkv, 0, len2);
    return true;
  };
  // Page ids of a unit's window, one logical page per lane: the raw table entry (an index that
  // must not be read is replaced by entry 0 of the row, which exists) and a ballot of the lanes
  // whose logical page may be read; an entry is checked against the pool when it is taken, so
  // nothing waits for the table load before the sub-tile that needs it.
  auto unit_pages = [&](const Unit& u, unsigned long long& okm) {
    const int lp = u.k_begin / kPage + 2 * u.w0 + lane;
    const bool ok = lp < a.max_pages && lp * kPage < u.seq_len;
    okm = __builtin_amdgcn_ballot_w64(ok);
    return a.page_table[(size_t)u.b * a.max_pages + (ok ? lp : 0)];
  };
  auto page_at = [&](int raw, unsigned long long okm, int i) {
    const int p = __builtin_amdgcn_readlane(raw, i);
    return ((okm >> i) & 1) && p >= 0 && p < a.num_pages ? p : -1;
  };
  // (the lane's part of the address is formed here from the lane id behind an empty asm, so it
  // is not hoisted into a register kept, and spilled, across the loop)
  auto load_q_of = [&](typename F::Q (&qq)[NB], int qb, int kvh, bool real) {
    int lid = lane;
    asm volatile("" : "+v"(lid));
    const char* qbase = a.q + ((size_t)qb * a.hq + kvh * a.group) * (size_t)ROWB;
#pragma unroll
    for (int cq = 0; cq < NB; ++cq) {
      const int hl = cq * 16 + (lid & 15);   // head within the group
      const char* row = real && hl < a.group ? qbase + (unsigned)(hl * ROWB) : zero_rows;
      F::load_q(qq[cq], row, lid >> 4);
    }
  };

  struct Buf {
    KOp k[2][NKS];
    VRow v[8];
  };
  Unit u = make_unit(b, j, I0 % a.hkv, 0, len0), un;
  unsigned long long pgm = 0, pgmn = 0;
  int pg = unit_pages(u, pgm), pgn = 0;
  typename F::Q qf[NB];
  load_q_of(qf, u.b, u.kvh, true);
  // K and V bases of the current unit's KV head and of the next unit's
  const char* kbase = a.k_cache + u.kvh * head_stride;
  const char* vbase = a.v_cache + u.kvh * head_stride;
  const char* kbase_n = kbase;
  const char* vbase_n = vbase;
  RowState<D> st[NB];
  int lo_wave = 0;   // some row of the wave has its split's peaked flag set (wave-uniform)
  bool has_next = false;
  // sub-tile t of unit u; t == u.nw is sub-tile 0 of the next unit when `next`, else (and when
  // there is none) the stand-ins
  auto fetch = [&](Buf& buf, int t, bool next) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int page = t < u.nw ? page_at(pg, pgm, (2 * t + kb) & 63)
                                : (next && has_next ? page_at(pgn, pgmn, kb) : -1);
      const char* kp = page >= 0 ? (t < u.nw ? kbase : kbase_n) + (size_t)page * page_stride : nan_rows;
      const char* vp = page >= 0 ? (t < u.nw ? vbase : vbase_n) + (size_t)page * page_stride : zero_rows;
      // (K and V are read once per call: non-temporal loads, which keep them from displacing
      // other lines in the caches, stream measurably faster)
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2) buf.k[kb][s2] = F::k_op_nt(kp + c * ROWB, s2, g);
#pragma unroll
      for (int i = 4 * kb; i < 4 * kb + 4; ++i)
        buf.v[i] = F::v_row_nt(vp + (F::vkey(i, g) - 16 * kb) * ROWB, c);
    }
  };
  auto compute = [&](Buf& buf, int t) {
    const int key0 = u.k_begin + kSubTile * (u.w0 + t);
    const int pos = u.seq_len - 1;
    if (key0 + kSubTile > u.seq_len) {
      // stale slots past the sequence end: V rows become zero, scores are masked below
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (key0 + F::vkey(i, g) >= u.seq_len) buf.v[i] = F::zero_v();
    }
    int posv[NB];
    bool lov[NB];
    const bool lo = needs_lo(pos);
#pragma unroll
    for (int cq = 0; cq < NB; ++cq) {
      posv[cq] = pos;
      lov[cq] = lo;
    }
    auto getK = [&](int kb, int s2) { return buf.k[kb][s2]; };
    auto getV = [&](int x) {
      if constexpr (std::is_same<E, float>::value) return buf.v[x];
      else return F::pack_v(buf.v, x);      // row block x, head dim NM c + x
    };
    subtile_step<E, D, NB>(st, qf, posv, getK, getV, a.cscale, key0, g, u.w0 + t == 0,
                                  key0 + kSubTile - 1 > pos, lov, lo, lo_wave);
  };
  // Every sub-tile of unit u, its first one already in flight in b0. Even sub-tiles are
  // computed from b0 and odd ones from b1; the next unit's first sub-tile goes to b0, during
  // the last compute when that is from b1 (an even count), else right after it.
  Buf b0, b1;
  auto run = [&]() {
    for (int t = 0;; t += 2) {
      fetch(b1, t + 1, false);
      compute(b0, t);
      if (t + 1 >= u.nw) {
        fetch(b0, t + 1, true);
        return;
      }
      fetch(b0, t + 2, true);
      compute(b1, t + 1);
      if (t + 2 >= u.nw) return;
    }
  };

  fetch(b0, 0, false);
  for (;;) {
    has_next = next_unit(u, un);
    if (has_next) pgn = unit_pages(un, pgmn);
    if (has_next) {
      kbase_n = a.k_cache + un.kvh * head_stride;
      vbase_n = a.v_cache + un.kvh * head_stride;
    }
    if constexpr (APPEND) {
      // Page update of the sequence's new token (position seq_len - 1), in the unit that holds
      // it: each lane that loads part of the token's K or V row in the unit's loop first copies
      // exactly those bytes from k_new / v_new into the slot, so its own later loads of them
      // (same lane, same address, in program order) see the token. No other wave reads the
      // slot. A slot without a page is skipped (its sub-tile reads the stand-in rows). When the
      // token is in the unit's first sub-tile, that sub-tile, loaded before the copy, is loaded
      // again.
      const int rel = u.seq_len - 1 - u.k_begin;          // offset in the split
      const int nt = rel / kSubTile - u.w0;               // sub-tile of the unit
      if (rel < split_len(a, u.seq_len) && nt >= 0 && nt < u.nw) {
        const int nk = rel - kSubTile * (u.w0 + nt), sl = nk & 15;
        const size_t src = ((size_t)u.b * a.hkv + u.kvh) * ROWB;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int page = page_at(pg, pgm, (2 * nt + kb) & 63);
          if ((nk >> 4) == kb && page >= 0) {
            char* ks = const_cast<char*>(kbase) + (size_t)page * page_stride + (size_t)sl * ROWB;
            char* vs = const_cast<char*>(vbase) + (size_t)page * page_stride + (size_t)sl * ROWB;
            if (c == sl) {
#pragma unroll
              for (int s2 = 0; s2 < NKS; ++s2) F::store_k(ks, s2, g, F::k_op(a.k_new + src, s2, g));
            }
#pragma unroll
            for (int i = 4 * kb; i < 4 * kb + 4; ++i)
              if (F::vkey(i, g) - 16 * kb == sl) F::store_v(vs, c, F::v_row(a.v_new + src, c));
            if (nt == 0) fetch(b0, 0, false);
          }
        }
      }
    }
    run();
    // q of the next unit, into registers the last compute no longer needs (its latency overlaps
    // the partial's stores; the next unit's first loads are already in flight)
    if (has_next && (un.b != u.b || un.kvh != u.kvh)) load_q_of(qf, un.b, un.kvh, true);
    if (u.w0 + u.nw >= u.nsub) {
      // Partial of split u.j: the accumulators of the group's heads are one contiguous block
      // of the workspace, written through the wave's LDS slice in whole 1 KB stores (each lane
      // holds 4 NM scattered-by-row values; stored directly they would be 16-byte pieces). The
      // lane's addresses are formed here from the lane id behind an empty asm: hoisted, they
      // would be registers kept (and spilled) across the loop, and a reload waits for every load
      // in flight.
      int lid = lane;
      asm volatile("" : "+v"(lid));
#pragma unroll
      for (int cq = 0; cq < NB; ++cq) {
        const int hl = cq * 16 + (lid & 15);
        float* lrow = lds_part + hl * D + 4 * (lid >> 4) * NM;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int mb = 0; mb < NM; mb += 4)
            *(f32x4*)(lrow + r * NM + mb) = f32x4{st[cq].acc[mb][r], st[cq].acc[mb + 1][r],
                                                  st[cq].acc[mb + 2][r], st[cq].acc[mb + 3][r]};
        const float rl = row_l(st[cq]);
        if ((lid >> 4) == 0 && hl < a.group)
          a.ws_ml[part_index(a, (size_t)u.b * a.hq + u.kvh * a.group + hl, u.j)] = make_float2(st[cq].m, rl);
      }
      // (non-temporal stores, like the K/V loads: measurably faster, and the combine reads the
      // partials at the same speed)
      char* dst = (char*)(a.ws_acc + part_index(a, (size_t)u.b * a.hq + u.kvh * a.group, u.j) * D);
      for (int i = lid; i < a.group * (D / 4); i += 64)
        __builtin_nontemporal_store(*(const f32x4*)(lds_part + 4 * i), (f32x4*)(dst + (unsigned)i * 16u));
    }
    if (!has_next) break;
    u = un;
    pg = pgn;
    pgm = pgmn;
    kbase = kbase_n;
    vbase = vbase_n;
  }
}

// Combine for rows of at most 32 splits. The partials of one (sequence, KV head) and split are a
// contiguous [group][D] block; a wave owns 256 consecutive floats of that block (lane: four
// floats of one row), folds them over the splits in ascending j and writes A / L. The
// accumulator loads run U splits ahead of the fold in a ring of U register slots (slot u holds
// split j with j % U == u; a slot is refilled as soon as it is folded), the first few before the
// row's split count is known; every split's (m, l) pair is loaded with its accumulators. Loads
// past the last split re-read it and are not folded, so every step issues the same loads.
template <int D, int U>
__global__ __launch_bounds__(kThreads) void combine_kernel(AttnParams a) {
  constexpr int FPL = 4;
  const int lane = threadIdx.x & 63;
  const int gw = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kWaves + (threadIdx.x >> 6)));
  const int G = a.group;
  const int chunks = (G * D + 64 * FPL - 1) / (64 * FPL);   // waves per (sequence, KV head)
  const int rg = gw / chunks, q = gw - rg * chunks;         // rg = b Hkv + kvh
  if (rg >= a.batch * a.hkv) return;
  const int b = rg / a.hkv;
  const int f = 64 * FPL * q + FPL * lane;                  // float of the [G][D] block
  if (f >= G * D) return;
  const int hl = f / D, d0 = f - hl * D;
  float* o = a.out + ((size_t)rg * G + hl) * D + d0;         // row b Hq + kvh G + hl
  const size_t blk0 = (size_t)rg * a.jmax * G;              // split 0 of the row group
  const float2* ml = a.ws_ml + blk0 + hl;
  const float* acc = a.ws_acc + blk0 * D + f;
  const size_t ml_step = G, acc_step = (size_t)G * D;
  const int seq_len = a.seq_lens[b];
  float2 mlj[U];
  f32x4 accj[U];
  // the first kEarly loads go out with the length's; the rest of the ring once the row's split
  // count J is known (clamped to its last split, so no load reads another row's slots)
  constexpr int kEarly = 4;
#pragma unroll
  for (int u = 0; u < kEarly; ++u) {
    const int jj = min(u, a.jmax - 1);
    mlj[u] = ml[jj * ml_step];
    accj[u] = *(const f32x4*)(acc + jj * acc_step);
  }
  const bool bad = seq_len <= 0 || seq_len > a.max_seq_len;
  const int J = bad ? 1 : (seq_len - 1) / split_len(a, seq_len) + 1;
#pragma unroll
  for (int u = kEarly; u < U; ++u) {
    const int jj = min(u, J - 1);
    mlj[u] = ml[jj * ml_step];
    accj[u] = *(const f32x4*)(acc + jj * acc_step);
  }
  if (bad) {
#pragma unroll
    for (int e = 0; e < FPL; ++e) o[e] = __builtin_nanf("");
    return;
  }
  float M = -__builtin_inff(), L = 0.f;
  float A[FPL];
#pragma unroll
  for (int e = 0; e < FPL; ++e) A[e] = 0.f;
  for (int j0 = 0; j0 < J; j0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u < J) {
        float fa, fb;
        fold_scalars(M, L, mlj[u].x, mlj[u].y, fa, fb);
        const f32x4 x = accj[u];
#pragma unroll
        for (int e = 0; e < FPL; ++e) A[e] = fold_elem(A[e], x[e], fa, fb);
      }
      const int jn = min(j0 + u + U, J - 1);
      mlj[u] = ml[jn * ml_step];
      accj[u] = *(const f32x4*)(acc + jn * acc_step);
    }
  }
  f32x4 r;
#pragma unroll
  for (int e = 0; e < FPL; ++e) r[e] = A[e] / L;
  *(f32x4*)o = r;
}

// Combine for long rows (more than 32 splits). The fold of a row is one sequential chain per
// element, and with one wave doing both a row's (m, l) fold and its elements' folds, every split
// cost the whole instruction stream of both. Here a workgroup owns one (sequence, q head) row and
// splits the chains among its waves, which run side by side: wave 0 runs the row's lazy reference
// M (fold_raises) and then forms a window's coefficients a, b lane-parallel with fold_scalars
// itself (lane u: split 64 w + u, from its m and the reference before it), so they carry the bits
// of the one-wave fold; it hands them over through LDS, one 64-split window at a time (two
// buffers, one barrier per window). Wave 1 runs L = fma(l, b, L a) as fold_scalars does, and wave
// 2 + e folds floats [64 e, 64 e + 64) of the row with fold_elem, its accumulator loads 64 splits
// ahead in a register ring. The output is A / L.
template <int D>
__global__ __launch_bounds__(64 * (D / 64 + 2)) void combine_rows_kernel(AttnParams a) {
  __shared__ float4 coef[2][64];   // [buffer][split of the window] (a, b, l, -)
  __shared__ float lrow;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int G = a.group;
  // Workgroups go to the 8 XCDs in turn (workgroup i to XCD i % 8); the rows are dealt out so
  // that XCD x takes the contiguous rows [x C, x C + C), C = ceil(rows / 8): the rows of one
  // (sequence, KV head) share the 128-byte lines of their (m, l) pairs, which one L2 then fetches
  // once. Workgroups past the last row exit.
  const int nrows = a.batch * a.hq;
  const int per_xcd = (nrows + 7) / 8;
  const int row = (int)(blockIdx.x % 8u) * per_xcd + (int)(blockIdx.x / 8u);   // b Hq + h
  if (row >= nrows) return;                                 // (the whole workgroup)
  const int rg = row / G, hl = row - rg * G, b = rg / a.hkv;
  const size_t blk0 = (size_t)rg * a.jmax * G;              // split 0 of the row group
  float* o = a.out + (size_t)row * D;
  const int seq_len = a.seq_lens[b];
  if (seq_len <= 0 || seq_len > a.max_seq_len) {
    if (wave > 1) o[64 * (wave - 2) + lane] = __builtin_nanf("");
    return;
  }
  const int J = (seq_len - 1) / split_len(a, seq_len) + 1;
  const int nw = (J + 63) / 64;
  if (wave == 0) {
    const float2* ml = a.ws_ml + blk0 + hl;                // split j at ml[j G]
    float M = -__builtin_inff();
    float2 mw = ml[(size_t)min(lane, J - 1) * G];
    for (int w = 0; w < nw; ++w) {
      const float2 mn = ml[(size_t)min(64 * (w + 1) + lane, J - 1) * G];
      const int cnt = min(64, J - 64 * w);
      float mprev = M;                                      // lane u: the reference before split 64 w + u
      auto chain = [&](auto full) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 64; ++u) {
          if (decltype(full)::value || u < cnt) {
            const float m = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mw.x), u));
            mprev = lane == u ? M : mprev;
            M = fold_raises(M, m) ? m : M;
          }
        }
      };
      if (cnt == 64) chain(std::true_type{});
      else chain(std::false_type{});
      // this lane's split's coefficients, from the same inputs as the chain's
      float Mu = mprev, Lu = 0.f, fa, fb;
      fold_scalars(Mu, Lu, mw.x, mw.y, fa, fb);
      coef[w & 1][lane] = make_float4(fa, fb, mw.y, 0.f);
      __syncthreads();
      mw = mn;
    }
    __syncthreads();
  } else if (wave == 1) {
    float L = 0.f;
    for (int w = 0; w < nw; ++w) {
      __syncthreads();                                      // window w's coefficients are in coef[w & 1]
      const float4 c = coef[w & 1][lane];
      const int cnt = min(64, J - 64 * w);
#pragma unroll
      for (int u = 0; u < 64; ++u) {
        if (u < cnt) {
          const float fa = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.x), u));
          const float fb = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.y), u));
          const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c.z), u));
          L = __builtin_fmaf(l, fb, L * fa);
        }
      }
    }
    if (lane == 0) lrow = L;
    __syncthreads();
  } else {
    const int e = wave - 2;
    // split j of this lane's float at byte j S + 4 lane of the wave's base (S = G D 4 bytes);
    // offsets fit 32 bits (the launcher checks jmax S)
    const char* base = (const char*)(a.ws_acc + (blk0 + hl) * D + 64 * e);
    const unsigned S = (unsigned)(G * D * 4), last = (unsigned)(J - 1) * S, lo = 4u * (unsigned)lane;
    auto ld = [&](unsigned off) { return *(const float*)(base + (off + lo)); };
    float ring[64];
    unsigned off = 0;
#pragma unroll
    for (int u = 0; u < 64; ++u) {
      ring[u] = ld(min(off, last));
      off += S;
    }
    float A = 0.f;
    for (int w = 0; w < nw; ++w) {
      __syncthreads();                                      // window w's coefficients are in coef[w & 1]
      const int cnt = min(64, J - 64 * w);
      auto fold = [&](auto full) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 64; ++u) {
          if (decltype(full)::value || u < cnt) {
            const float2 c = *(const float2*)&coef[w & 1][u];   // (a, b), the same in every lane
            A = fold_elem(A, ring[u], c.x, c.y);
          }
          ring[u] = ld(min(off, last));
          off += S;
        }
      };
      if (cnt == 64) fold(std::true_type{});
      else fold(std::false_type{});
    }
    __syncthreads();                                        // wave 1's L is in lrow
    o[64 * e + lane] = A / lrow;
  }
}

// ------------------------------------------------------------------------------------------
// Prefill: a workgroup owns a tile of query columns (token-major: column = token * G + head)
// of one (sequence, KV head) and walks every 32-key sub-tile that any of its rows needs, in
// ascending order, folding each finished split into the row state. K/V sub-tiles are staged
// in LDS and shared by all NW waves (the global loads of the next NPF sub-tiles are in flight
// while one is computed); each wave holds NBW column blocks. The row accumulator A, touched
// only when a split ends, lives in registers (AREG) or in LDS. For bf16 the PV operand
// comes from the row-major V sub-tile through transposing LDS reads, which puts head dim
// d = 16 mb + 4 g + r in accumulator (mb, r) of lane group g; for fp32 the layout is the
// decode one, d = NM (4 g + r) + mb.
template <int D, typename E> struct Lds {
  static constexpr int ROWB = D * (int)sizeof(E);
  static constexpr int STRIDE = ROWB + 32;              // row pitch: conflict-free K and V reads
  static constexpr int TILE = kSubTile * STRIDE;        // one K or V sub-tile
};
constexpr int kPageCache = 2048;

// Longest-first order of the prefill work. A work item is (sequence b, query tile t); its cost
// is its sub-tile count n(b, t) = (first_pos + min((t + 1) tq, n_new) + 31) / 32, which never
// decreases with t. Workgroup rank i takes the i-th item in the order (n descending, then b
// ascending, then t ascending), so the longest tiles start first and the short ones fill the
// end of the grid. Which workgroup computes an item never changes its numbers.
struct PfSeq {
  int q0;          // first row of q and out
  int len;         // keys of the sequence (seq_lens[b], or the dense row range)
  int fp, n, nt;   // first position, rows of q and out (n_new, clipped to total_tokens), tiles
  bool bad;        // invalid sequence: its tiles cost nothing and only write NaN rows
};
// A sequence is invalid when its q_starts pair is out of order, starts outside q or ends past
// total_tokens, has more new tokens than max_q_len or than its length, or its length or (dense)
// key rows are out of range. Its rows that lie in q (rows q0 .. min(q1, total_tokens) - 1, none
// when the pair is out of order or starts outside q) come out NaN; other sequences' rows are
// untouched.
__device__ __forceinline__ PfSeq pf_seq(const AttnParams& a, int b, int tq) {
  PfSeq s{0, 0, 0, 0, 0, false};
  if (b >= a.batch) return s;
  const int q0 = a.q_starts[b], q1 = a.q_starts[b + 1];
  if (q0 < 0 || q1 < q0 || q0 >= a.total_tokens) return s;
  int len;
  bool rows_ok = true;
  if (a.k_starts) {
    const int k0 = a.k_starts[b], k1 = a.k_starts[b + 1];
    len = k1 - k0;
    rows_ok = k0 >= 0 && k1 <= a.k_rows;
  } else {
    len = a.seq_lens[b];
  }
  const int n_new = q1 - q0;
  s.q0 = q0;
  s.len = len;
  s.n = min(q1, a.total_tokens) - q0;
  // tiles, at most max_q_len / tq per sequence, so the grid always holds every item (an
  // invalid sequence with more rows covers them in strides; a valid one is never capped)
  s.nt = min((s.n + tq - 1) / tq, (a.max_q_len + tq - 1) / tq);
  s.bad = q1 > a.total_tokens || n_new > a.max_q_len || len > a.max_seq_len || n_new > len || !rows_ok;
  s.fp = len - n_new;
  return s;
}
// tiles of the sequence whose sub-tile count exceeds K (K >= -1): n(b, t) > K exactly when
// min((t + 1) tq, n_new) >= 32 K + 1 - first_pos
// (tq = 2^lg: the group size divides 128)
__device__ __forceinline__ int pf_tiles_above(const PfSeq& s, int K, int lg) {
  if (s.nt <= 0) return 0;
  if (s.bad) return K < 0 ? s.nt : 0;
  const int R = 32 * K + 1 - s.fp;
  if (R > s.n) return 0;
  return s.nt - (R <= 0 ? 0 : ((R + (1 << lg) - 1) >> lg) - 1);
}
// Item of rank i for this wave (wave-uniform); false when i is past the last item.
__device__ bool pf_item(const AttnParams& a, int tq, int i, int& ob, int& otile) {
  const int lane = threadIdx.x & 63;
  const int lg = __builtin_ctz(tq);
  const int chunks = (a.batch + 63) / 64;
  const PfSeq s0 = pf_seq(a, lane, tq);   // the first 64 sequences stay in registers
  auto seq_of = [&](int ch) { return ch == 0 ? s0 : pf_seq(a, 64 * ch + lane, tq); };
  auto count_above = [&](int K) {
    int c = 0;
    for (int ch = 0; ch < chunks; ++ch) c += wave_sum_i(pf_tiles_above(seq_of(ch), K, lg));
    return __builtin_amdgcn_readfirstlane(c);
  };
  if (i >= count_above(-1)) return false;
  // smallest K with count_above(K) <= i: the cost of item i
  int lo = -1, hi = (a.max_seq_len + 31) / 32;
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (count_above(mid) <= i) hi = mid;
    else lo = mid;
  }
  int r = i - count_above(hi);   // rank among the items of cost hi, in (b, t) order
  for (int ch = 0; ch < chunks; ++ch) {
    const PfSeq s = seq_of(ch);
    const int ge = pf_tiles_above(s, hi - 1, lg), gt = pf_tiles_above(s, hi, lg);
    const int e = ge - gt;   // tiles t in [nt - ge, nt - gt) cost exactly hi
    const int incl = wave_incl_scan(e, lane);
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(incl > r);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const int before = __shfl(incl - e, l);
      ob = __builtin_amdgcn_readfirstlane(64 * ch + l);
      otile = __builtin_amdgcn_readfirstlane(__shfl(s.nt - ge, l) + (r - before));
      return true;
    }
    r -= __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  return false;
}

template <typename E, int D, int NBW, int NW, bool RING, int NPF, bool AREG, int MINB, bool DENSE>
__global__ __launch_bounds__(64 * NW, MINB) void prefill_kernel(AttnParams a) {
  using F = Frag<E, D>;
  using LD = Lds<D, E>;
  constexpr bool BF = std::is_same<E, __bf16>::value;
  constexpr int NM = D / 16;
  constexpr int NT = 64 * NW;
  constexpr int COLS = NW * NBW * 16;
  constexpr int CHUNKS = LD::ROWB / 16;                  // 16-byte chunks per row
  constexpr int PAIRS = kSubTile * CHUNKS;               // (row, chunk) slots of a sub-tile
  constexpr int PP = (PAIRS + NT - 1) / NT;
  // bf16, D 128: K/V sub-tiles go from HBM straight into LDS (global_load_lds_dwordx4, 16 bytes
  // per lane, lane i of an instruction to byte 16 i of its 1 KB block), double-buffered, in an
  // unpadded layout whose 16-byte chunks are rotated per row (chunk lc of row R at chunk
  // (lc + 2 R) % 16): the same banks as a 32-byte row padding, which the K reads and the
  // transposing V reads use without conflicts.
  // Otherwise the sub-tile is staged through registers into one padded buffer.
  constexpr bool DMA = BF && D == 128 && (NW == 4 || NW == 8) && NPF == 1;
  constexpr int KPS = 2;                                   // sub-tiles per DMA step
  constexpr int DTILE = KPS * kSubTile * LD::ROWB;         // 16 KB: 64 keys
  __shared__ __attribute__((aligned(16))) char lds_kv[2][DMA ? 16 : LD::TILE];
  // the two buffers are separate variables, so the compiler can tell that the reads of one
  // do not wait for the transfers into the other
  __shared__ __attribute__((aligned(16))) char lds_d0[2][DMA ? DTILE : 16];   // [K, V]
  __shared__ __attribute__((aligned(16))) char lds_d1[2][DMA ? DTILE : 16];
  __shared__ f32x4 lds_A[AREG ? 1 : NW][AREG ? 1 : NBW][AREG ? 1 : NM][64];   // [wave][block][row block][lane]
  __shared__ int lds_pages[kPageCache];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int G = a.group;
  const int tq = COLS / G;                       // tokens per tile (G divides COLS)
  // workgroup = (item rank, KV head); items longest first
  const int kvh = (int)(blockIdx.x % (unsigned)a.hkv);
  int b = 0, tile = 0;
  if (!pf_item(a, tq, (int)(blockIdx.x / (unsigned)a.hkv), b, tile)) return;
  const PfSeq sq = pf_seq(a, b, tq);
  const int q0 = sq.q0;
  const int n_new = sq.n;                 // rows of this sequence in q and out
  const int t0 = tile * tq;
  // dense: the sequence's keys are rows k0 .. k0 + seq_len - 1 of [k_rows][Hkv][D] arrays
  const int k0 = DENSE ? a.k_starts[b] : 0;
  const int seq_len = sq.len;
  const bool bad_seq = sq.bad;
  const int first_pos = sq.fp;
  if (bad_seq) {
    // an invalid sequence: NaN rows only; its tiles (at most max_q_len / tq of them) cover
    // rows t0 + k * (tiles * tq), k = 0, 1, ..., of every column
    const int rstep = sq.nt * tq;
#pragma unroll
    for (int cb = 0; cb < NBW; ++cb) {
      const int col = (wave * NBW + cb) * 16 + c;
      for (int tok = t0 + col / G; tok < n_new; tok += rstep) {
        float* dst = a.out + ((size_t)(q0 + tok) * a.hq + kvh * G + col % G) * D + g * (D / 4);
#pragma unroll
        for (int i = 0; i < D / 16; ++i) *(f32x4*)(dst + 4 * i) = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      }
    }
    return;
  }
  const int t_last = min(t0 + tq, n_new) - 1;
  const int pos_max_wg = first_pos + t_last;
  const int S = split_len(a, seq_len);
  const size_t head_stride = (size_t)kPage * LD::ROWB;
  const size_t page_stride = (size_t)a.hkv * head_stride;
  // bytes between consecutive keys of one KV head in HBM (paged: rows of a page; dense: rows of
  // the [k_rows][Hkv][D] arrays), and the offset of logical page lp (16 keys) from the head base
  const int rstride = DENSE ? a.hkv * LD::ROWB : LD::ROWB;
  auto page_off = [&](int page) -> size_t {
    return DENSE ? (size_t)(k0 + kPage * page) * (size_t)rstride : (size_t)(unsigned)max(page, 0) * page_stride;
  };

  typename F::Q qf[NBW];
  RowState<D> st[NBW];
  float Mrow[NBW], Lrow[NBW];
  f32x4 Areg[AREG ? NBW : 1][NM];
  int pos_c[NBW], blk_max[NBW];
  bool valid_c[NBW];
  int wave_min = 0x7fffffff, wave_max = -1;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int col0 = (wave * NBW + cb) * 16;
    const int col = col0 + c;
    const int tok = t0 + col / G;
    valid_c[cb] = tok < n_new && !bad_seq;
    pos_c[cb] = valid_c[cb] ? first_pos + tok : -1;
    const int tok_lo = t0 + col0 / G, tok_hi = min(t0 + (col0 + 15) / G, n_new - 1);
    blk_max[cb] = (tok_lo < n_new && !bad_seq) ? first_pos + tok_hi : -1;
    if (tok_lo < n_new && !bad_seq) {
      wave_min = min(wave_min, first_pos + tok_lo);
      wave_max = max(wave_max, first_pos + tok_hi);
    }
    if (valid_c[cb]) {
      const char* row = a.q + ((size_t)(q0 + tok) * a.hq + kvh * G + col % G) * (size_t)LD::ROWB;
      F::load_q(qf[cb], row, g);
    } else {
      F::zero_q(qf[cb]);
    }
    Mrow[cb] = -__builtin_inff();
    Lrow[cb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) Areg[AREG ? cb : 0][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // position part of the P_lo choice (the positions are fixed for the whole tile)
  bool lo_c[NBW], lo_any_c = false;
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    lo_c[cb] = needs_lo(pos_c[cb]);
    lo_any_c = lo_any_c || lo_c[cb];
  }
  const bool lo_w = wave_any(lo_any_c);
  int lo_wave = 0;   // some row of the wave has its split's peaked flag set (wave-uniform)
  const int nsub = bad_seq ? 0 : (pos_max_wg + kSubTile) / kSubTile;
  // page ids of the logical pages the tile reads, in an LDS ring of kPageCache entries
  // (logical page lp in slot lp % kPageCache), refilled half a ring ahead of use
  const int npg_total = nsub * (kSubTile / kPage);
  if constexpr (!DMA && !DENSE) {
    for (int i = threadIdx.x; i < min(npg_total, kPageCache); i += NT) lds_pages[i] = page_of(a, b, i, seq_len);
    __syncthreads();
  }

  // staging: each thread owns the same (row, 16-byte chunk) slots of the K and V sub-tiles
  const char* kbase = a.k_cache + kvh * (DENSE ? (size_t)LD::ROWB : head_stride);
  const char* vbase = a.v_cache + kvh * (DENSE ? (size_t)LD::ROWB : head_stride);
  // A ring of NPF register sets keeps NPF sub-tiles of loads in flight. The loop is unrolled
  // by NPF so every set has a fixed name, and every stage issues exactly the same loads, so
  // the wait before each LDS store counts exactly the later loads. Absent pages and sub-tiles
  // past the end read kNanRows (K) and kZeroRows (V), and so do V rows at or past seq_len:
  // no stale cache bytes reach an MFMA, and a row that needs an absent page comes out NaN.
  u32x4 preK[NPF][PP], preV[NPF][PP];
  const int last = nsub - 1;   // sub-tiles past it (and every one when nsub == 0) read stand-ins
  const char* nan_rows = (const char*)&kNanRows;
  const char* zero_rows = (const char*)kZeroRows;
  // this thread's slots: row r of the sub-tile (key key0 + r, in page half r / kPage) and the
  // byte offset of its 16-byte chunk inside a page
  unsigned srow[PP], sin_page[PP];
#pragma unroll
  for (int k = 0; k < PP; ++k) {
    const unsigned pair = (unsigned)min((int)threadIdx.x + k * NT, PAIRS - 1);
    const unsigned r = pair / CHUNKS, ch = pair - r * CHUNKS;
    srow[k] = r;
    sin_page[k] = (r % kPage) * LD::ROWB + ch * 16;
  }
  // When the rows of each slot lie in one page (a page's row chunks are a multiple of the
  // thread count), the page id and the K address are wave-uniform (scalar registers).
  constexpr bool UNI = (kPage * CHUNKS) % NT == 0;
  // page id of slot k of sub-tile u (-1: none), read from the LDS ring one step before the
  // loads that use it, so that the read's latency is not on the path of every step
  auto page_at = [&](int u, int k) {
    const unsigned half = UNI ? (unsigned)(k * NT / (kPage * CHUNKS)) : srow[k] / kPage;
    const unsigned lp = 2u * (unsigned)u + half;
    if constexpr (DENSE) return u <= last && (int)lp * kPage < seq_len ? (int)lp : -1;
    else return u <= last ? lds_pages[lp % kPageCache] : -1;
  };
  int pgq[PP];
  auto stage_load = [&](int u, const int (&pgs)[PP], u32x4 (&pk)[PP], u32x4 (&pv)[PP]) {
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      int page = pgs[k];
      if (UNI) page = __builtin_amdgcn_readfirstlane(page);
      const bool vin = u * kSubTile + (int)srow[k] < seq_len;
      if constexpr (DENSE) {
        // rows at or past seq_len are another sequence's (or past the arrays): stand-ins
        const bool in = page >= 0 && vin;
        const size_t off = page_off(page) + (size_t)(srow[k] % kPage) * (unsigned)(rstride - LD::ROWB);
        pk[k] = *(const u32x4*)((in ? kbase + off : nan_rows) + sin_page[k]);
        pv[k] = *(const u32x4*)((in ? vbase + off : zero_rows) + sin_page[k]);
      } else {
        const size_t off = page_off(page);
        const char* kp = page >= 0 ? kbase + off : nan_rows;
        const char* vp = page >= 0 && vin ? vbase + off : zero_rows;
        pk[k] = *(const u32x4*)(kp + sin_page[k]);
        pv[k] = *(const u32x4*)(vp + sin_page[k]);
      }
    }
  };
  auto stage_store = [&](const u32x4 (&pk)[PP], const u32x4 (&pv)[PP]) {
#pragma unroll
    for (int k = 0; k < PP; ++k) {
      const int pair = threadIdx.x + k * NT;
      if (pair < PAIRS) {
        const int r = pair / CHUNKS, ch = pair - r * CHUNKS;
        *(u32x4*)(&lds_kv[0][r * LD::STRIDE + ch * 16]) = pk[k];
        *(u32x4*)(&lds_kv[1][r * LD::STRIDE + ch * 16]) = pv[k];
      }
    }
  };

  // DMA layout: physical chunk of logical chunk lc in row R, and this lane's byte offsets of the
  // K operand of k-step s2 (row 16 kb + c, chunk 4 s2 + g; key block kb adds 16 rows) and of
  // the V operand of row block x (rows rv and rv + 16, chunk 2 x + ((c & 3) >> 1), byte
  // 8 (c & 1) in it)
  auto pchunk = [](int lc, int R) { return (lc + 2 * R) & 15; };
  unsigned koff[NM / 2], voff[NM];
  const int rv = 4 * g + (c >> 2);
#pragma unroll
  for (int s2 = 0; s2 < NM / 2; ++s2) koff[s2] = c * LD::ROWB + (pchunk(4 * s2 + g, c) << 4);
#pragma unroll
  for (int x = 0; x < NM; ++x)
    voff[x] = rv * LD::ROWB + (pchunk(2 * x + ((c & 3) >> 1), rv) << 4) + 8 * (c & 1);
  // one sub-tile step: compute sub-tile u from the K/V tile at kt / vt, then fold split j into
  // the row state when u ends it
  // (sub-tiles come in ascending order: split j and the sub-tile's place in it are counted)
  const int SS = S / kSubTile;
  int sj = 0, sr = 0;
  auto step = [&](int u, const char* kt, const char* vt) __attribute__((always_inline)) {
    const int key0 = u * kSubTile;
    const int j = sj;
    const bool first = sr == 0;
    const bool last_of_split = sr == SS - 1 || u + 1 == nsub;
    if (++sr == SS) {
      sr = 0;
      ++sj;
    }
    if (wave_max >= key0) {
      auto getK = [&](int kb, int s2) {
        if constexpr (DMA) return *(const u32x4*)(kt + koff[s2] + kb * 16 * LD::ROWB);
        else return F::k_op(kt + (16 * kb + c) * LD::STRIDE, s2, g);
      };
      auto getV = [&](int x) {
        if constexpr (DMA) return F::v_tr_at(vt + voff[x], 16 * LD::ROWB);
        else if constexpr (BF) return F::v_tr(vt, LD::STRIDE, x, c, g);
        else return F::v_row(vt + F::vkey(x, g) * LD::STRIDE, c);
      };
      // all blocks advance together; on the diagonal of the tile the mask leaves rows whose
      // position is below key0 as they are (see subtile_step)
      subtile_step<E, D, NBW, BF>(st, qf, pos_c, getK, getV, a.cscale, key0, g, first,
                                  key0 + kSubTile - 1 > wave_min, lo_c, lo_w, lo_wave);
    }
    if (last_of_split && wave_max >= j * S) {
      // fold split j into the rows of every block that reaches it (also when this wave's rows
      // ended before this last sub-tile of the split). A row whose position is below the
      // split's first key holds the empty state there, which the fold leaves as it was, so
      // every lane folds.
#pragma unroll
      for (int cb = 0; cb < NBW; ++cb) {
        if (blk_max[cb] < j * S) continue;
        float fa, fb;
        // the product A a of fold_elem() is A itself in every lane that keeps its reference
        // (a = 1), so it is formed only when some lane of the wave raises (rarely past split 0)
        const bool scale = wave_any(fold_raises(Mrow[cb], st[cb].m));
        fold_scalars(Mrow[cb], Lrow[cb], st[cb].m, row_l(st[cb]), fa, fb);
        if (AREG) {
          if (scale) {
#pragma unroll
            for (int mb = 0; mb < NM; ++mb) Areg[AREG ? cb : 0][mb] = Areg[AREG ? cb : 0][mb] * fa;
          }
#pragma unroll
          for (int mb = 0; mb < NM; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              Areg[AREG ? cb : 0][mb][e] = __builtin_fmaf(st[cb].acc[mb][e], fb, Areg[AREG ? cb : 0][mb][e]);
        } else {
#pragma unroll
          for (int mb = 0; mb < NM; ++mb) {
            f32x4& slot = lds_A[AREG ? 0 : wave][AREG ? 0 : cb][AREG ? 0 : mb][lane];
            f32x4 A = j > 0 ? slot : f32x4{0.f, 0.f, 0.f, 0.f};   // (LDS slots start unwritten)
#pragma unroll
            for (int e = 0; e < 4; ++e) A[e] = fold_elem(A[e], st[cb].acc[mb][e], fa, fb);
            slot = A;
          }
        }
      }
    }
  };
  // when the page-id reads reach a new half of the ring (first page lpn), fill the half after
  // it; the slots it overwrites belong to pages no later read needs, and the end-of-step
  // barriers order the refill against the earlier readers and the later ones
  auto refill = [&](int lpn) {
    if (RING && !DENSE && lpn % (kPageCache / 2) == 0 && lpn >= kPageCache / 2) {
      const int base = lpn + kPageCache / 2;
      for (int t = threadIdx.x; t < kPageCache / 2; t += NT)
        if (base + t < npg_total) lds_pages[(base + t) % kPageCache] = page_of(a, b, base + t, seq_len);
    }
  };

  if constexpr (DMA) {
    // A step covers KPS = 2 sub-tiles (64 keys, 4 pages). This wave's TPW 1 KB blocks of each
    // step's tile: rows R = RPW wave + 4 t + lane / 16, all in page PG of the step, lane's chunk
    // at physical position lane % 16.
    constexpr int RPW = KPS * kSubTile / NW, TPW = RPW / 4;
    const int PG = RPW * wave / kPage;
    unsigned soff[TPW];
    int srw[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      const int R = RPW * wave + 4 * t + (lane >> 4), Rp = R & 15;
      srw[t] = R;
      soff[t] = Rp * rstride + (((lane - 2 * Rp) & 15) << 4);   // logical chunk of physical lane % 16
    }
    // Page ids: lane i of pg_cur holds the page this wave reads in step pbase + i (logical page
    // 4 (pbase + i) + PG, in sub-tile 2 (pbase + i) + PG / 2; -1 when that sub-tile is past the
    // last one or the page must not be read), pg_nxt the next 64 steps' ids; a step takes its id
    // with one readlane, so no memory wait sits between the steps' loads.
    auto pg_batch = [&](int base) {
      if constexpr (DENSE) return 0;
      const int sp = base + lane;
      const int p = page_of_nb(a, b, 4 * sp + PG, seq_len);
      return 2 * sp + (PG >> 1) <= last ? p : -1;
    };
    int pbase = 0;
    int pg_cur = pg_batch(0), pg_nxt = pg_batch(64);
    typedef __attribute__((address_space(3))) void* lds_ptr;
    typedef const __attribute__((address_space(1))) char* gptr;
    auto dma = [&](int sp, char (&dst)[2][DMA ? DTILE : 16]) __attribute__((always_inline)) {
      int page;
      if constexpr (DENSE) {
        // no table: logical page 4 sp + PG, absent past the last sub-tile or the sequence end
        const int lp = 4 * sp + PG;
        page = 2 * sp + (PG >> 1) <= last && lp * kPage < seq_len ? lp : -1;
      } else {
        page = __builtin_amdgcn_readlane(pg_cur, sp - pbase);
        if (sp - pbase == 63) {
          pbase += 64;
          pg_cur = pg_nxt;
          pg_nxt = pg_batch(pbase + 64);
        }
      }
      const size_t off = page_off(page);
      if (page >= 0 && (4 * sp + PG + 1) * kPage <= seq_len) {
        // the whole page lies before seq_len: one scalar base per page, lane offsets
        const gptr kp = (gptr)(kbase + off), vp = (gptr)(vbase + off);
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          // (the offset is taken here, so the loads address with scalar base + 32-bit offset)
          unsigned o = soff[t];
          asm volatile("" : "+v"(o));
          __builtin_amdgcn_global_load_lds(kp + o, (lds_ptr)&dst[0][(TPW * wave + t) * 1024], 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vp + o, (lds_ptr)&dst[1][(TPW * wave + t) * 1024], 16, 0, 0);
        }
      } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          const bool vin = sp * KPS * kSubTile + srw[t] < seq_len;
          const char *kp, *vp;
          if constexpr (DENSE) {
            // rows at or past seq_len belong to another sequence (or lie past the arrays): both
            // K and V read stand-ins there, at the stand-ins' own row pitch
            const bool in = page >= 0 && vin;
            const unsigned std_off = soff[t] - (unsigned)(srw[t] & 15) * (unsigned)(rstride - LD::ROWB);
            kp = in ? kbase + off + soff[t] : nan_rows + std_off;
            vp = in ? vbase + off + soff[t] : zero_rows + std_off;
          } else {
            kp = (page >= 0 ? kbase + off : nan_rows) + soff[t];
            vp = (page >= 0 && vin ? vbase + off : zero_rows) + soff[t];
          }
          __builtin_amdgcn_global_load_lds((gptr)kp, (lds_ptr)&dst[0][(TPW * wave + t) * 1024], 16, 0, 0);
          __builtin_amdgcn_global_load_lds((gptr)vp, (lds_ptr)&dst[1][(TPW * wave + t) * 1024], 16, 0, 0);
        }
      }
    };
    auto steps = [&](int sp, char (&buf)[2][DMA ? DTILE : 16]) __attribute__((always_inline)) {
      step(KPS * sp, buf[0], buf[1]);
      if (KPS * sp + 1 < nsub) step(KPS * sp + 1, buf[0] + kSubTile * LD::ROWB, buf[1] + kSubTile * LD::ROWB);
    };
    // (s_waitcnt vmcnt(0) alone: the tile's HBM -> LDS transfers of this wave have landed)
    constexpr int kWaitVm0 = 0x0F70;
    const int nst = (nsub + KPS - 1) / KPS;
    dma(0, lds_d0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    // step sp from buffer sp % 2 while sp + 1 lands in the other (unrolled by two, so every
    // buffer access names its variable)
    for (int sp = 0; sp < nst; sp += 2) {
      if (sp + 1 < nst) dma(sp + 1, lds_d1);
      steps(sp, lds_d0);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (sp + 1 >= nst) break;
      if (sp + 2 < nst) dma(sp + 2, lds_d0);
      steps(sp + 1, lds_d1);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
  } else {
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
#pragma unroll
    for (int k = 0; k < PP; ++k) pgq[k] = page_at(i, k);
    stage_load(i, pgq, preK[i], preV[i]);
  }
#pragma unroll
  for (int k = 0; k < PP; ++k) pgq[k] = page_at(NPF, k);
  for (int u0 = 0; u0 < nsub; u0 += NPF) {
#pragma unroll
  for (int i = 0; i < NPF; ++i) {
    const int u = u0 + i;
    if (u >= nsub) break;
    refill((u + NPF) * (kSubTile / kPage));
    stage_store(preK[i], preV[i]);
    __syncthreads();
    stage_load(u + NPF, pgq, preK[i], preV[i]);
#pragma unroll
    for (int k = 0; k < PP; ++k) pgq[k] = page_at(u + NPF + 1, k);
    step(u, lds_kv[0], lds_kv[1]);
    __syncthreads();
  }
  }
  }
  // Epilogue: out = A / L for every valid row.
#pragma unroll
  for (int cb = 0; cb < NBW; ++cb) {
    const int col = (wave * NBW + cb) * 16 + c;
    const int tok = t0 + col / G;
    if (tok >= n_new) continue;
    float* dst = a.out + ((size_t)(q0 + tok) * a.hq + kvh * G + col % G) * D;
    const bool ok = valid_c[cb];
    f32x4 R[NM];
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) {
      const f32x4 A = AREG ? Areg[AREG ? cb : 0][mb] : lds_A[AREG ? 0 : wave][AREG ? 0 : cb][AREG ? 0 : mb][lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) R[mb][e] = ok ? A[e] / Lrow[cb] : __builtin_nanf("");
    }
    if constexpr (BF) {
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) *(f32x4*)(dst + 16 * mb + 4 * g) = R[mb];
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int m4 = 0; m4 < NM / 4; ++m4)
          *(f32x4*)(dst + NM * (4 * g + r) + 4 * m4) =
              f32x4{R[4 * m4][r], R[4 * m4 + 1][r], R[4 * m4 + 2][r], R[4 * m4 + 3][r]};
    }
  }
}

// ------------------------------------------------------------------------------------------
// Page update: one wave per new token. The wave finds the token's sequence with one ballot per
// 64 sequences (the count of q_starts[b] <= t; q_starts ascending), then copies the token's K
// and V rows of every KV head into its page slot, 16 bytes per lane.
template <int ROWB>
__global__ __launch_bounds__(256) void page_update_kernel(const char* k_new, const char* v_new,
                                                          const int32_t* q_starts,
                                                          const int32_t* seq_lens,
                                                          const int32_t* page_table,
                                                          int max_pages, int num_pages, int batch,
                                                          int total_tokens, int hkv,
                                                          char* k_cache, char* v_cache) {
  constexpr int CH = ROWB / 16;
  const int lane = threadIdx.x & 63;
  const int t0 = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  const int first = q_starts[0], end = q_starts[batch];
  // up to 64 sequences: every lane holds q_starts[lane] and seq_lens[lane], loaded with the
  // token rows, so the page id is one load after them
  const bool small = batch <= 64;
  const int qs_l = small && lane <= batch ? q_starts[lane] : 0;
  const int sl_l = small && lane < batch ? seq_lens[lane] : 0;
  for (int t = t0; t < total_tokens; t += (int)gridDim.x * 4) {
    if (t < first || t >= end) continue;
    // the token's first 64 chunks are loaded before its page is known
    const bool l0 = lane < hkv * CH;
    const int h0 = lane / CH, ch0 = lane - h0 * CH;
    const size_t src0 = ((size_t)t * hkv + (l0 ? h0 : 0)) * ROWB + (l0 ? ch0 : 0) * 16;
    const u32x4 k0 = *(const u32x4*)(k_new + src0);
    const u32x4 v0 = *(const u32x4*)(v_new + src0);
    int bq, s0, s1, len;                            // bq: last b with q_starts[b] <= t
    if (small) {
      bq = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < batch && qs_l <= t)) - 1;
      s0 = __builtin_amdgcn_readlane(qs_l, bq);
      s1 = bq + 1 < 64 ? __builtin_amdgcn_readlane(qs_l, bq + 1) : end;
      len = __builtin_amdgcn_readlane(sl_l, bq);
    } else {
      int cnt = 0;
      for (int c0 = 0; c0 < batch; c0 += 64) {
        const int i = c0 + lane;
        cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i < batch && q_starts[i] <= t));
      }
      bq = cnt - 1;
      s0 = q_starts[bq];
      s1 = q_starts[bq + 1];
      len = seq_lens[bq];
    }
    if (t >= s1) continue;                          // q_starts not ascending: not a token of bq
    const int pos = len - (s1 - s0) + (t - s0);
    if (pos < 0) continue;
    const int lp = pos / kPage;
    if (lp >= max_pages) continue;
    const int page = page_table[(size_t)bq * max_pages + lp];
    if (page < 0 || page >= num_pages) continue;
    const size_t slot = ((size_t)page * hkv * kPage + (pos % kPage)) * ROWB;   // head 0 row
    if (l0) {
      const size_t dst = slot + (size_t)h0 * kPage * ROWB + ch0 * 16;
      *(u32x4*)(k_cache + dst) = k0;
      *(u32x4*)(v_cache + dst) = v0;
    }
    for (int i = lane + 64; i < hkv * CH; i += 64) {
      const int h = i / CH, ch = i - h * CH;
      const size_t src = ((size_t)t * hkv + h) * ROWB + ch * 16;
      const size_t dst = slot + (size_t)h * kPage * ROWB + ch * 16;
      const u32x4 kv = *(const u32x4*)(k_new + src);
      const u32x4 vv = *(const u32x4*)(v_new + src);
      *(u32x4*)(k_cache + dst) = kv;
      *(u32x4*)(v_cache + dst) = vv;
    }
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
  if (c->split_policy != BI_SPLIT_FIXED && c->split_policy != BI_SPLIT_BY_BATCH &&
      c->split_policy != BI_SPLIT_BY_BATCH_FILL)
    return BI_EINVAL;
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
  // by-batch: at most ceil(k CUs / (batch Hkv)) splits (k = 2, or 8 to fill the resident
  // waves), and never more than ceil(len / 32)
  const int64_t b = batch > 0 ? batch : 1;
  const int64_t k = c->split_policy == BI_SPLIT_BY_BATCH_FILL ? 8 : 2;
  const int64_t by_batch = (k * (int64_t)cu_count() + b * c->num_kv_heads - 1) / (b * c->num_kv_heads);
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
  a.num_cus = c->split_policy != BI_SPLIT_FIXED ? cu_count() : 0;
  return a;
}

int launched() { return hipGetLastError() == hipSuccess ? BI_OK : BI_EHIP; }

// Decode grid: as many workgroups as the device keeps resident at once, but no more than there
// can be items.
template <typename E, int D, int NB, bool APPEND>
int launch_partials_nb(const AttnParams& a, hipStream_t s) {
  constexpr int NWV = DecWaves<E, NB>::value;
  static int per_cu_cache[64];   // resident workgroups per CU, per device (benign race)
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  int per_cu = (dev >= 0 && dev < 64) ? per_cu_cache[dev] : 0;
  if (per_cu <= 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_split_kernel<E, D, NB, APPEND>, 64 * NWV, 0) !=
            hipSuccess || per_cu <= 0)
      per_cu = 1;
    (void)hipGetLastError();
    if (dev >= 0 && dev < 64) per_cu_cache[dev] = per_cu;
  }
  // up to one workgroup per item: a small batch spreads over as many CUs as it has items (one
  // CU's own bandwidth is the limit there), a large one fills every resident slot
  const int64_t items_max = (int64_t)a.batch * a.hkv * a.jmax;
  int64_t wgs = std::min<int64_t>((int64_t)cu_count() * per_cu, items_max);
  wgs = std::max<int64_t>(wgs, 1);
  hipLaunchKernelGGL((decode_split_kernel<E, D, NB, APPEND>), dim3((unsigned)wgs), dim3(64 * NWV), 0, s, a);
  return launched();
}

template <typename E, int D, bool APPEND>
int launch_partials(const AttnParams& a, hipStream_t s) {
  if (a.group <= 16) return launch_partials_nb<E, D, 1, APPEND>(a, s);
  if (a.group == 32) return launch_partials_nb<E, D, 2, APPEND>(a, s);
  return launch_partials_nb<E, D, 4, APPEND>(a, s);
}

// Combine: up to 32 splits per row, one wave per 256 floats with four floats per lane and every
// split's loads issued at once; beyond, one workgroup per row (combine_rows_kernel), whose
// element waves address a row group's partials with 32-bit offsets (decode_params refuses a call
// whose row group would pass 2 GiB of partials).
template <int D>
void launch_combine_d(const AttnParams& a, hipStream_t s) {
  if (a.jmax <= 32) {
    const int64_t waves = (int64_t)a.batch * a.hkv * ((a.group * D + 255) / 256);
    const dim3 grid((unsigned)((waves + kWaves - 1) / kWaves));
    hipLaunchKernelGGL((combine_kernel<D, 32>), grid, dim3(kThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((combine_rows_kernel<D>), dim3((unsigned)((a.batch * a.hq + 7) / 8 * 8)), dim3(64 * (D / 64 + 2)), 0, s, a);
  }
}
int launch_combine(const AttnParams& a, int D, hipStream_t s) {
  if (D == 128) launch_combine_d<128>(a, s);
  else launch_combine_d<64>(a, s);
  return launched();
}

// Validates a decode call and fills the parameters; BI_OK when there is work to launch.
int decode_params(const bi_attn_cfg* cfg, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                  const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out,
                  const void* workspace, size_t workspace_bytes, bool need_kv, bool need_out,
                  AttnParams* a) {
  int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || max_seq_len < 0 || max_pages < 0 || num_pages < 0) return BI_EINVAL;
  if (batch == 0) return -1;   // nothing to do
  if (!seq_lens || max_seq_len == 0) return BI_EINVAL;
  if (need_kv && (!q || !k_cache || !v_cache || !page_table || max_pages == 0 || num_pages == 0))
    return BI_EINVAL;
  if (need_kv && (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))) return BI_EINVAL;
  if (need_out && (!out || !aligned16(out))) return BI_EINVAL;
  // the row-parallel combine addresses one (sequence, KV head)'s partials with 32-bit offsets
  if (jmax_of(cfg, batch, max_seq_len) * (cfg->num_q_heads / cfg->num_kv_heads) * cfg->head_dim * 4 >=
      ((int64_t)1 << 31))
    return BI_EUNSUPPORTED;
  const size_t need = ws_bytes(cfg, batch, batch, max_seq_len);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return BI_EWORKSPACE;
  *a = base_params(cfg);
  a->q = (const char*)q;
  a->k_cache = (const char*)k_cache;
  a->v_cache = (const char*)v_cache;
  a->page_table = page_table;
  a->seq_lens = seq_lens;
  a->out = out;
  a->max_pages = max_pages;
  a->num_pages = num_pages;
  a->batch = batch;
  a->total_tokens = batch;
  a->max_q_len = 1;
  a->max_seq_len = max_seq_len;
  a->jmax = (int32_t)jmax_of(cfg, batch, max_seq_len);
  a->ws_ml = (float2*)workspace;
  a->ws_acc = (float*)((char*)workspace + ws_ml_bytes((int64_t)batch * cfg->num_q_heads, a->jmax));
  return BI_OK;
}

template <bool APPEND>
int dispatch_partials(const bi_attn_cfg* cfg, const AttnParams& a, hipStream_t s) {
  const bool bf = cfg->dtype == BI_BF16;
  if (cfg->head_dim == 128)
    return bf ? launch_partials<__bf16, 128, APPEND>(a, s) : launch_partials<float, 128, APPEND>(a, s);
  return bf ? launch_partials<__bf16, 64, APPEND>(a, s) : launch_partials<float, 64, APPEND>(a, s);
}

// Validates the new-token arguments of an appending decode and adds them to the parameters.
int append_params(const bi_attn_cfg* cfg, const void* k_new, const void* v_new, AttnParams* a) {
  (void)cfg;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return BI_EINVAL;
  a->k_new = (const char*)k_new;
  a->v_new = (const char*)v_new;
  return BI_OK;
}

// bf16: two workgroups of 4 waves per CU (their barriers are independent, so one fills the
// other's stalls), 2 column blocks per wave, A in registers, one staging set in flight (the
// other workgroup's loads cover the latency). fp32: one workgroup of 4 waves, A in LDS.
template <typename E, int D, bool DENSE = false>
int launch_prefill(const AttnParams& a, hipStream_t s) {
  constexpr bool BF = std::is_same<E, __bf16>::value;
  constexpr int NW = 4, NBW = 2, NPF = BF ? 1 : 4, MINB = BF ? 2 : 1;
  constexpr bool AREG = BF;
  // sequences longer than the LDS page-id ring need the kernel that refills it (paged layout)
  const bool ring = !DENSE && (int64_t)a.max_seq_len + kSubTile > (int64_t)kPageCache * kPage;
  const int tq = NW * NBW * 16 / a.group;
  // one workgroup per (tile, KV head): every sequence has at most ceil(max_q_len / tq) tiles,
  // so the grid holds every item; workgroups past the real item count exit at once
  const int64_t wgs = (int64_t)((a.max_q_len + tq - 1) / tq) * a.batch * a.hkv;
  if (wgs > 0x7fffffff) return BI_EUNSUPPORTED;
  const dim3 grid((unsigned)wgs);
  if (ring) hipLaunchKernelGGL((prefill_kernel<E, D, NBW, NW, true, NPF, AREG, MINB, false>), grid, dim3(64 * NW), 0, s, a);
  else hipLaunchKernelGGL((prefill_kernel<E, D, NBW, NW, false, NPF, AREG, MINB, DENSE>), grid, dim3(64 * NW), 0, s, a);
  return launched();
}

// Allocation-free decode: the split partials live in a static device array of
// BI_NOALLOC_SCRATCH_BYTES (each device the library runs on holds its own copy until the
// process ends). Host code never names the array as an address: the device address is
// queried once per device with hipGetSymbolAddress (the device current at the call) and kept.
static __device__ __attribute__((aligned(256))) unsigned char scratch[BI_NOALLOC_SCRATCH_BYTES];

void* scratch_ptr() {
  static void* ptrs[64];   // per device (benign race: every caller stores the same address)
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptrs[dev] = p;
  }
  return ptrs[dev];
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
  const int64_t waves = std::min<int64_t>(total_tokens, 65536);   // one wave per token (strided)
  const unsigned blocks = (unsigned)((waves + 3) / 4);
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
  AttnParams a;
  const int st = decode_params(cfg, q, k_cache, v_cache, page_table, max_pages, num_pages, seq_lens,
                               batch, max_seq_len, out, workspace, workspace_bytes, true, true, &a);
  if (st != BI_OK) return st < 0 ? BI_OK : st;
  if (dispatch_partials<false>(cfg, a, stream) != BI_OK) return BI_EHIP;
  return launch_combine(a, cfg->head_dim, stream);
}

int bi_attn_decode_noalloc(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* page_table, int32_t max_pages,
                           int32_t num_pages, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float* out, hipStream_t stream) {
  const int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || max_seq_len < 0) return BI_EINVAL;
  if (batch == 0) return BI_OK;
  if (ws_bytes(cfg, batch, batch, max_seq_len) > (size_t)BI_NOALLOC_SCRATCH_BYTES) return BI_EWORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return BI_EHIP;
  // every partial the combine reads is written by the partials kernel of the same call first,
  // so nothing needs clearing between calls
  return bi_attn_decode(cfg, q, k_cache, v_cache, page_table, max_pages, num_pages, seq_lens, batch,
                        max_seq_len, out, ws, (size_t)BI_NOALLOC_SCRATCH_BYTES, stream);
}

int bi_attn_decode_partials(const bi_attn_cfg* cfg, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* page_table, int32_t max_pages,
                            int32_t num_pages, const int32_t* seq_lens, int32_t batch,
                            int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  AttnParams a;
  const int st = decode_params(cfg, q, k_cache, v_cache, page_table, max_pages, num_pages, seq_lens,
                               batch, max_seq_len, nullptr, workspace, workspace_bytes, true, false, &a);
  if (st != BI_OK) return st < 0 ? BI_OK : st;
  return dispatch_partials<false>(cfg, a, stream);
}

int bi_attn_decode_append_partials(const bi_attn_cfg* cfg, const void* q, const void* k_new,
                                   const void* v_new, void* k_cache, void* v_cache,
                                   const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnParams a;
  int st = decode_params(cfg, q, k_cache, v_cache, page_table, max_pages, num_pages, seq_lens,
                         batch, max_seq_len, nullptr, workspace, workspace_bytes, true, false, &a);
  if (st != BI_OK) return st < 0 ? BI_OK : st;
  if ((st = append_params(cfg, k_new, v_new, &a)) != BI_OK) return st;
  return dispatch_partials<true>(cfg, a, stream);
}

int bi_attn_decode_append(const bi_attn_cfg* cfg, const void* q, const void* k_new,
                          const void* v_new, void* k_cache, void* v_cache,
                          const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                          const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnParams a;
  int st = decode_params(cfg, q, k_cache, v_cache, page_table, max_pages, num_pages, seq_lens,
                         batch, max_seq_len, out, workspace, workspace_bytes, true, true, &a);
  if (st != BI_OK) return st < 0 ? BI_OK : st;
  if ((st = append_params(cfg, k_new, v_new, &a)) != BI_OK) return st;
  if (dispatch_partials<true>(cfg, a, stream) != BI_OK) return BI_EHIP;
  return launch_combine(a, cfg->head_dim, stream);
}

int bi_attn_decode_combine(const bi_attn_cfg* cfg, const int32_t* seq_lens, int32_t batch,
                           int32_t max_seq_len, float* out, const void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  AttnParams a;
  const int st = decode_params(cfg, nullptr, nullptr, nullptr, nullptr, 0, 0, seq_lens, batch,
                               max_seq_len, out, workspace, workspace_bytes, false, true, &a);
  if (st != BI_OK) return st < 0 ? BI_OK : st;
  return launch_combine(a, cfg->head_dim, stream);
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

int bi_attn_varlen(const bi_attn_cfg* cfg, const void* q, const void* k, const void* v,
                   const int32_t* q_starts, const int32_t* k_starts, int32_t batch, int32_t total_q,
                   int32_t total_k, int32_t max_q_len, int32_t max_seq_len, float* out,
                   hipStream_t stream) {
  int st = check_cfg(cfg);
  if (st != BI_OK) return st;
  if (batch < 0 || total_q < 0 || total_k < 0 || max_q_len < 0 || max_seq_len < 0) return BI_EINVAL;
  if (batch == 0 || total_q == 0 || max_q_len == 0) return BI_OK;
  if (!q || !k || !v || !q_starts || !k_starts || !out) return BI_EINVAL;
  if (max_seq_len == 0 || total_k == 0) return BI_EINVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return BI_EINVAL;
  AttnParams a = base_params(cfg);
  a.q = (const char*)q;
  a.k_cache = (const char*)k;
  a.v_cache = (const char*)v;
  a.q_starts = q_starts;
  a.k_starts = k_starts;
  a.k_rows = total_k;
  a.out = out;
  a.batch = batch;
  a.total_tokens = total_q;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  const bool bf = cfg->dtype == BI_BF16;
  if (cfg->head_dim == 128)
    return bf ? launch_prefill<__bf16, 128, true>(a, stream) : launch_prefill<float, 128, true>(a, stream);
  return bf ? launch_prefill<__bf16, 64, true>(a, stream) : launch_prefill<float, 64, true>(a, stream);
}

}  // extern "C"
