// core.hpp — the invariant arithmetic shared by the decode and prefill kernels (gfx950).
//
// Bit contract. A query token's output depends only on its own q, its position, the keys
// 0..pos and the fixed split size S. Everything that touches its numbers lives in this file
// and runs identically in both kernels:
//   * keys are reduced in splits [jS, jS+S) of absolute positions, each split in 32-key
//     sub-tiles in ascending order (the fixed split size of neican.ai insight page, section
//     技术原理与创新点解析, batch-invariant attention item);
//   * inside a sub-tile, QK^T and PV are MFMA contractions on v_mfma_f32_16x16x32_bf16
//     (bf16 data) or v_mfma_f32_16x16x4_f32 (fp32 data), with one fixed operand layout;
//   * the softmax state (m, l, acc) of a split is reset at the split start and folded into
//     the row state (M, L, A) in ascending split order by fold_scalars()/fold_elem().
// Kernels differ only in where operand bytes come from (HBM or LDS) and in which rows share
// a wave; the registers handed to the MFMAs are byte-identical either way.
//
// Layout (one 64-lane wave, lane = c + 16 g, c in 0..15, g in 0..3). The query rows of a
// "column block" are the N dimension of every MFMA, so each lane owns one query row c:
//   S^T[key][c] = K[key] . q[c]    A = K (rows = 16 keys),       B = q^T (cols = 16 queries)
//   O^T[d][c]  += V^T[d][key] P    A = V^T (rows = 16 dims),     B = P^T (cols = 16 queries)
// The C layout of a 16x16 MFMA puts rows 4g..4g+3 of column c in lane (c, g), so the scores,
// probabilities and accumulators of query c never leave lanes {c, c+16, c+32, c+48}: the row
// max and row sum are a two-step xor butterfly over those lanes, the same in every lane.
// Head dimension d sits in PV row block mb = d % NM at row d / NM (NM = D / 16), so a lane
// loads NM contiguous V elements per key and ends with the contiguous output range
// d in [4 g NM, 4 g NM + 4 NM):   acc[mb][r] <-> d = NM (4 g + r) + mb.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#pragma clang fp contract(off)

namespace bi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kSubTile = 32;   // keys per sub-tile: two 16-key MFMA row blocks
constexpr int kPage = 16;      // tokens per KV page

__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// exp2 on the transcendental unit (v_exp_f32): exp2(-inf) = +0, exp2(0) = 1.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
// x + partner is commutative, so every lane of the group ends with the same bits.
__device__ __forceinline__ float xor_sum(float v) {
  v = v + __shfl_xor(v, 16);
  v = v + __shfl_xor(v, 32);
  return v;
}

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ unsigned bf16_pack2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (unsigned)__builtin_bit_cast(unsigned short, a) |
         ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
}
__device__ __forceinline__ float bf16_lo_f(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_f(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// ------------------------------------------------------------------------------------------
// Per-dtype operand fragments. `E` is the storage type of q/k/v (bf16 or float).
template <typename E, int D> struct Frag;

// bf16: QK^T in D/32 k-steps of v_mfma_f32_16x16x32_bf16. Lane (c, g) holds, for k-step s,
// dims [32 s + 8 g, 32 s + 8 g + 8) of its row (query c for B, key c of the block for A).
// PV: one k-step covers the sub-tile's 32 keys; slot i of lane group g is key
// 4 g + i (i < 4) or 16 + 4 g + i - 4 (i >= 4), which is exactly where the C layout of the
// two score blocks left P, so P never moves between lanes.
template <int D> struct Frag<__bf16, D> {
  static constexpr int NKS = D / 32;
  static constexpr int NM = D / 16;
  static constexpr int ROWB = D * 2;                 // bytes per K/V row
  struct Q { u32x4 v[NKS]; };
  struct K { u32x4 v[2][NKS]; };
  struct V { u32x4 v[NM]; };                         // A operand of PV per row block mb
  // Raw V: for each of the lane's 8 keys, dims [NM c, NM c + NM).
  using VRow = typename std::conditional<NM == 8, u32x4, u32x2>::type;
  struct VRaw { VRow v[8]; };

  __device__ static inline int vkey(int i, int g) { return (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4); }

  __device__ static inline void load_q(Q& q, const char* row, int g) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) q.v[s] = *(const u32x4*)(row + (32 * s + 8 * g) * 2);
  }
  __device__ static inline void zero_q(Q& q) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) q.v[s] = u32x4{0, 0, 0, 0};
  }
  // A-operand rows of key block kb: `row` points at the K row of key 16 kb + c.
  __device__ static inline void load_k_block(K& k, int kb, const char* row, int g) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) k.v[kb][s] = *(const u32x4*)(row + (32 * s + 8 * g) * 2);
  }
  __device__ static inline void zero_k_block(K& k, int kb) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) k.v[kb][s] = u32x4{0, 0, 0, 0};
  }
  // `row` points at the V row of key vkey(i, g).
  __device__ static inline void load_v_key(VRaw& r, int i, const char* row, int c) {
    r.v[i] = *(const VRow*)(row + NM * c * 2);
  }
  __device__ static inline void zero_v_key(VRaw& r, int i) { r.v[i] = VRow{}; }
  // Transpose raw V into the A operand of each row block: slot pair (2p, 2p+1) of block mb
  // holds dim NM c + mb of keys vkey(2p), vkey(2p+1). Pure data movement.
  __device__ static inline void pack_v(V& v, const VRaw& r) {
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) {
      const int w = mb >> 1;
      unsigned out[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const unsigned a = r.v[2 * p][w], b = r.v[2 * p + 1][w];
        out[p] = (mb & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      v.v[mb] = u32x4{out[0], out[1], out[2], out[3]};
    }
  }
  __device__ static inline void qk(f32x4 s[2], const K& k, const Q& q) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NKS; ++st) a = mma_bf16(k.v[kb][st], q.v[st], a);
      s[kb] = a;
    }
  }
  // acc += P V with P = P_hi + P_lo, both bf16 (round to nearest even), hi first.
  __device__ static inline void pv(f32x4 acc[NM], const V& v, const float p[2][4]) {
    unsigned hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = p[i >> 1][(2 * i) & 3], x1 = p[i >> 1][(2 * i + 1) & 3];
      hi[i] = bf16_pack2(x0, x1);
      lo[i] = bf16_pack2(x0 - bf16_lo_f(hi[i]), x1 - bf16_hi_f(hi[i]));
    }
    const u32x4 H = {hi[0], hi[1], hi[2], hi[3]}, L = {lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) {
      acc[mb] = mma_bf16(v.v[mb], H, acc[mb]);
      acc[mb] = mma_bf16(v.v[mb], L, acc[mb]);
    }
  }
};

// fp32: QK^T in D/4 k-steps of v_mfma_f32_16x16x4_f32; lane (c, g) holds dim (D/4) g + s of
// k-step s. PV in 8 k-steps (kb, r): slot g is key 16 kb + 4 g + r, the lane's own score.
template <int D> struct Frag<float, D> {
  static constexpr int NKS = D / 4;
  static constexpr int NM = D / 16;
  static constexpr int ROWB = D * 4;
  struct Q { float v[NKS]; };
  struct K { float v[2][NKS]; };
  struct VRaw { float v[8][NM]; };   // key index kb*4 + r
  struct V { float v[8][NM]; };

  __device__ static inline int vkey(int i, int g) { return 16 * (i >> 2) + 4 * g + (i & 3); }

  __device__ static inline void load_q(Q& q, const char* row, int g) {
    const f32x4* p = (const f32x4*)(row + (NKS * g) * 4);
#pragma unroll
    for (int s = 0; s < NKS / 4; ++s) {
      const f32x4 t = p[s];
      q.v[4 * s] = t[0]; q.v[4 * s + 1] = t[1]; q.v[4 * s + 2] = t[2]; q.v[4 * s + 3] = t[3];
    }
  }
  __device__ static inline void zero_q(Q& q) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) q.v[s] = 0.f;
  }
  __device__ static inline void load_k_block(K& k, int kb, const char* row, int g) {
    const f32x4* p = (const f32x4*)(row + (NKS * g) * 4);
#pragma unroll
    for (int s = 0; s < NKS / 4; ++s) {
      const f32x4 t = p[s];
      k.v[kb][4 * s] = t[0]; k.v[kb][4 * s + 1] = t[1]; k.v[kb][4 * s + 2] = t[2]; k.v[kb][4 * s + 3] = t[3];
    }
  }
  __device__ static inline void zero_k_block(K& k, int kb) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) k.v[kb][s] = 0.f;
  }
  __device__ static inline void load_v_key(VRaw& r, int i, const char* row, int c) {
    const f32x4* p = (const f32x4*)(row + NM * c * 4);
#pragma unroll
    for (int s = 0; s < NM / 4; ++s) {
      const f32x4 t = p[s];
      r.v[i][4 * s] = t[0]; r.v[i][4 * s + 1] = t[1]; r.v[i][4 * s + 2] = t[2]; r.v[i][4 * s + 3] = t[3];
    }
  }
  __device__ static inline void zero_v_key(VRaw& r, int i) {
#pragma unroll
    for (int m = 0; m < NM; ++m) r.v[i][m] = 0.f;
  }
  __device__ static inline void pack_v(V& v, const VRaw& r) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int m = 0; m < NM; ++m) v.v[i][m] = r.v[i][m];
  }
  __device__ static inline void qk(f32x4 s[2], const K& k, const Q& q) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NKS; ++st) a = mma_f32(k.v[kb][st], q.v[st], a);
      s[kb] = a;
    }
  }
  __device__ static inline void pv(f32x4 acc[NM], const V& v, const float p[2][4]) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) acc[mb] = mma_f32(v.v[i][mb], p[i >> 2][i & 3], acc[mb]);
  }
};

// ------------------------------------------------------------------------------------------
// Softmax state of one query row (one lane group), in base-2 units: m is the running max of
// q.k * c with c = scale * log2(e); p = 2^(q.k c - m); l = sum p; acc = sum p v.
template <int D> struct RowState {
  static constexpr int NM = D / 16;
  float m, l;
  f32x4 acc[NM];
};

// One 32-key sub-tile of one column block.
//   first:   this is the first sub-tile of the split (state is reset, not rescaled)
//   mask:    some key of the sub-tile may lie after some row's position (wave-uniform)
//   partial: some row of the block must keep its state unchanged (wave-uniform)
//   key0:    absolute position of the sub-tile's first key; pos: this lane's row position
//   active:  key0 <= pos for this lane's row (only read when `partial`)
template <typename E, int D>
__device__ __forceinline__ void subtile_step(RowState<D>& st, const typename Frag<E, D>::Q& q,
                                             const typename Frag<E, D>::K& k,
                                             const typename Frag<E, D>::V& v, float cscale,
                                             int key0, int g, int pos, bool active, bool first,
                                             bool mask, bool partial) {
  using F = Frag<E, D>;
  constexpr int NM = D / 16;
  f32x4 s[2];
  F::qk(s, k, q);
  float x[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) x[kb][r] = s[kb][r];
  if (mask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        x[kb][r] = (key0 + 16 * kb + 4 * g + r <= pos) ? x[kb][r] : -__builtin_inff();
  }
  float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                   fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
  mx = xor_max(mx);
  const float mnew = first ? mx * cscale : fmaxf(st.m, mx * cscale);
  const float nm = -mnew;
  float p[2][4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) p[kb][r] = ex2(__builtin_fmaf(x[kb][r], cscale, nm));
  float rs = ((p[0][0] + p[0][1]) + (p[0][2] + p[0][3])) + ((p[1][0] + p[1][1]) + (p[1][2] + p[1][3]));
  rs = xor_sum(rs);
  f32x4 acc[NM];
  float lnew;
  if (first) {
    lnew = rs;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    const float alpha = ex2(st.m - mnew);
    lnew = __builtin_fmaf(st.l, alpha, rs);
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) acc[mb] = st.acc[mb] * alpha;
  }
  F::pv(acc, v, p);
  if (partial) {
    if (active) {
      st.m = mnew;
      st.l = lnew;
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) st.acc[mb] = acc[mb];
    }
  } else {
    st.m = mnew;
    st.l = lnew;
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) st.acc[mb] = acc[mb];
  }
}

// Ascending fold of split j's state into the row state (the same function the combine kernel
// applies element by element): M' = max(M, m), a = 2^(M - M'), b = 2^(m - M'),
// L = L a + l b, A = A a + acc b, with split 0 copied as is.
__device__ __forceinline__ void fold_scalars(float& M, float& L, float m, float l, bool first,
                                             float& a, float& b) {
  if (first) {
    M = m; L = l; a = 0.f; b = 1.f;
    return;
  }
  const float Mn = fmaxf(M, m);
  a = ex2(M - Mn);
  b = ex2(m - Mn);
  L = __builtin_fmaf(L, a, l * b);
  M = Mn;
}
__device__ __forceinline__ float fold_elem(float A, float acc, float a, float b, bool first) {
  return first ? acc : __builtin_fmaf(A, a, acc * b);
}

}  // namespace bi
