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

// Cross-lane exchanges for the row max and row sum, on the VALU (gfx950 lane swaps):
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with the even rows of
// its second, v_permlane32_swap the upper half of the first with the lower half of the second.
// Started from two copies of x, the pair (a, b) holds (x[l], x[l ^ 16]) resp. (x[l], x[l ^ 32])
// ordered the same way in both partner lanes. Written as the instructions themselves (the
// builtins' second result is not reliable in this compiler), with wait states around them.
// Their inputs are always VALU results, never MFMA results: the compiler inserts no MFMA
// wait states in front of an asm block.
__device__ __forceinline__ void swap_rows16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
// IEEE 754-2019 maximum (a NaN input gives NaN; -0 < +0): gfx950's v_maximum3_f32, which needs
// no canonicalising of its inputs. Kept as compiler-visible operations (not inline asm) because
// their inputs are MFMA results, and only the compiler inserts the wait states an MFMA result
// needs before a VALU instruction may read it.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
__device__ __forceinline__ float xor_max(float v) {
  float a = v, b = v;
  swap_rows16(a, b);
  v = vmax(a, b);
  a = v;
  b = v;
  swap_halves32(a, b);
  return vmax(a, b);
}
// Both partners add the same two values in the same order, so they get the same bits.
__device__ __forceinline__ float xor_sum(float v) {
  float a = v, b = v;
  swap_rows16(a, b);
  v = a + b;
  a = v;
  b = v;
  swap_halves32(a, b);
  return a + b;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two fp32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; lo in bits 0..15.
__device__ __forceinline__ unsigned bf16_pack2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// c plus the eight bf16 values of a lane's P words, one word (two values) at a time in word
// order, each with one v_dot2c_f32_bf16 against (1, 1): the products are exact and the pair's
// sum is added to c in fp32. Words of zeros leave c as it is.
// (The words are copied out of the vector by name before the bit_cast: a bit_cast of an
// indexed element of an ext_vector_type vector compiles to a read of element 0 here.)
__device__ __forceinline__ float add_words(float c, u32x4 w) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  const unsigned e[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, e[k]), one, c, false);
  return c;
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
  using KOp = u32x4;
  using VRow = typename std::conditional<NM == 8, u32x4, u32x2>::type;  // dims [NM c, NM c + NM)
  struct Q { u32x4 v[NKS]; };
  struct VRaw { VRow v[8]; };

  __device__ static inline int vkey(int i, int g) { return (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4); }
  // operand bytes of k-step st from a K (or q) row
  __device__ static inline KOp k_op(const char* row, int st, int g) {
    return *(const u32x4*)(row + (32 * st + 8 * g) * 2);
  }
  __device__ static inline KOp zero_k() { return u32x4{0, 0, 0, 0}; }
  // raw V chunk of lane column c from a V row
  __device__ static inline VRow v_row(const char* row, int c) { return *(const VRow*)(row + NM * c * 2); }
  // the same loads marked non-temporal (streaming: data read once, not kept in the caches)
  __device__ static inline KOp k_op_nt(const char* row, int st, int g) {
    return __builtin_nontemporal_load((const u32x4*)(row + (32 * st + 8 * g) * 2));
  }
  __device__ static inline VRow v_row_nt(const char* row, int c) {
    return __builtin_nontemporal_load((const VRow*)(row + NM * c * 2));
  }
  // the inverses of k_op and v_row: a lane's part of a K or V row back to memory
  __device__ static inline void store_k(char* row, int st, int g, KOp x) { *(u32x4*)(row + (32 * st + 8 * g) * 2) = x; }
  __device__ static inline void store_v(char* row, int c, VRow x) { *(VRow*)(row + NM * c * 2) = x; }
  __device__ static inline VRow zero_v() { return VRow{}; }
  __device__ static inline void load_q(Q& q, const char* row, int g) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) q.v[s] = k_op(row, s, g);
  }
  __device__ static inline void zero_q(Q& q) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) q.v[s] = zero_k();
  }
  // Each score block s[b][kb] accumulates its k-steps in ascending order; the 2 NB chains are
  // interleaved k-step by k-step so that consecutive MFMAs are independent. PIPE (operands
  // read from LDS): k-step 0 is read and waited for alone, then the reads of k-steps
  // [1, C) go out before the MFMAs of k-step 0 and those of [C, NKS) before the MFMAs of
  // [1, C) (C = 1 + NKS / 2), each batch after the previous one has landed, as in pv_pass.
  // Otherwise the reads of k-step st + 1 are issued before the MFMAs of k-step st.
  template <int NB, bool PIPE = false, class KGet>
  __device__ static inline void qk(f32x4 (&s)[NB][2], KGet& getK, const Q (&q)[NB]) {
#pragma unroll
    for (int b = 0; b < NB; ++b) s[b][0] = s[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (PIPE) {
      constexpr int C = 1 + NKS / 2;
      constexpr int kWaitLgkm0 = 0xC07F;   // s_waitcnt lgkmcnt(0) alone
      u32x4 k[NKS][2];
      auto mfmas = [&](int st) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          s[b][0] = mma_bf16(k[st][0], q[b].v[st], s[b][0]);
          s[b][1] = mma_bf16(k[st][1], q[b].v[st], s[b][1]);
        }
      };
      k[0][0] = getK(0, 0);
      k[0][1] = getK(1, 0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int st = 1; st < C; ++st) {
        k[st][0] = getK(0, st);
        k[st][1] = getK(1, st);
      }
      __builtin_amdgcn_sched_barrier(0);
      mfmas(0);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int st = C; st < NKS; ++st) {
        k[st][0] = getK(0, st);
        k[st][1] = getK(1, st);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 1; st < C; ++st) mfmas(st);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = C; st < NKS; ++st) mfmas(st);
      return;
    }
    u32x4 k0 = getK(0, 0), k1 = getK(1, 0);
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      u32x4 n0 = k0, n1 = k1;
      if (st + 1 < NKS) {
        n0 = getK(0, st + 1);
        n1 = getK(1, st + 1);
      }
      if (PIPE) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        s[b][0] = mma_bf16(k0, q[b].v[st], s[b][0]);
        s[b][1] = mma_bf16(k1, q[b].v[st], s[b][1]);
      }
      k0 = n0;
      k1 = n1;
    }
  }
  // acc += P_hi V and acc += P_lo V: P_hi = bf16(p), P_lo = bf16(p - P_hi) (round to nearest
  // even), P_lo zero in the lanes without lo_row, whose accumulators then keep their bits (an
  // exact zero added to a nonzero or +0 value), and the lo products skipped altogether (PIPE)
  // when no lane has lo_row. Every accumulator takes its hi MFMA before its lo MFMA, whether
  // the two are interleaved by row block or run as two passes, so the bits are the same.
  // getV(mb) returns the A operand of row block mb: 8 bf16 of one head-dim row d for the key
  // slots vkey(0..7, g). Which d a (row block, lane) holds is the caller's choice; each
  // output element's dot product is the same whichever MFMA row computes it.
  // PIPE (LDS operands): the operands of the first NPRE row blocks (vpre) were read by the caller
  // ahead of time; the other row blocks' reads go out in two batches, each issued right after
  // the previous batch has landed and before the MFMAs of that batch, which run while it lands.
  // (The compiler drains every outstanding LDS read at each wait here, so the waits are placed
  // explicitly where nothing newer is in flight.) Otherwise the reads of row block mb + 2 are
  // issued before the MFMAs of row block mb.
  static constexpr int NPRE = 2;
  template <int NB, bool PIPE, class VGet>
  __device__ static inline void pv_pass(f32x4 (&acc)[NB][NM], VGet& getV, const u32x4 (&P)[NB],
                                        const u32x4 (&vpre)[NPRE]) {
    if constexpr (PIPE) {
      constexpr int B1 = NPRE, B2 = NPRE + (NM - NPRE + 1) / 2;   // batches [0,B1) [B1,B2) [B2,NM)
      constexpr int kWaitLgkm0 = 0xC07F;                          // s_waitcnt lgkmcnt(0) alone
      u32x4 v[NM];
#pragma unroll
      for (int i = 0; i < B1; ++i) v[i] = vpre[i];
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int i = B1; i < B2; ++i) v[i] = getV(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = 0; mb < B1; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][mb] = mma_bf16(v[mb], P[b], acc[b][mb]);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
      for (int i = B2; i < NM; ++i) v[i] = getV(i);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = B1; mb < B2; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][mb] = mma_bf16(v[mb], P[b], acc[b][mb]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int mb = B2; mb < NM; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][mb] = mma_bf16(v[mb], P[b], acc[b][mb]);
    } else {
      u32x4 vf = getV(0), vf1 = getV(1);
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) {
        const u32x4 vn = mb + 2 < NM ? getV(mb + 2) : vf;
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][mb] = mma_bf16(vf, P[b], acc[b][mb]);
        vf = vf1;
        vf1 = vn;
      }
    }
  }
  // PIPE: vpre holds the operands of the first NPRE row blocks, read before the softmax so that
  // the first PV MFMAs need not wait for LDS.
  template <int NB, bool PIPE = false, class VGet>
  __device__ static inline void pv(f32x4 (&acc)[NB][NM], VGet& getV, const float (&p)[NB][2][4],
                                   float (&l)[NB], const bool (&lo_row)[NB], bool lo_any,
                                   const u32x4 (&vpre)[NPRE]) {
    u32x4 H[NB], L[NB];
    auto make_lo = [&](int b) {
      unsigned lo[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = p[b][i >> 1][(2 * i) & 3], x1 = p[b][i >> 1][(2 * i + 1) & 3];
        const unsigned h = H[b][i];
        lo[i] = lo_row[b] ? bf16_pack2(x0 - bf16_lo_f(h), x1 - bf16_hi_f(h)) : 0u;
      }
      L[b] = u32x4{lo[0], lo[1], lo[2], lo[3]};
    };
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      unsigned hi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) hi[i] = bf16_pack2(p[b][i >> 1][(2 * i) & 3], p[b][i >> 1][(2 * i + 1) & 3]);
      H[b] = u32x4{hi[0], hi[1], hi[2], hi[3]};
      l[b] = add_words(l[b], H[b]);
      if (!PIPE) {
        make_lo(b);
        l[b] = add_words(l[b], L[b]);
      }
    }
    if constexpr (PIPE) {
      // LDS operands: the hi pass, then (only when some row needs it) the lo pass
      pv_pass<NB, PIPE>(acc, getV, H, vpre);
      if (lo_any) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          make_lo(b);
          l[b] = add_words(l[b], L[b]);
        }
        asm volatile("" ::: "memory");   // the V operands are read again, not kept
        u32x4 vre[NPRE];
#pragma unroll
        for (int i = 0; i < NPRE; ++i) vre[i] = getV(i);
        pv_pass<NB, PIPE>(acc, getV, L, vre);
      }
    } else {
      // register operands (an HBM-bound caller): hi and lo MFMA per row block, P_lo zero in
      // the rows that do not need it
#pragma unroll
      for (int mb = 0; mb < NM; ++mb) {
        const u32x4 vf = getV(mb);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          acc[b][mb] = mma_bf16(vf, H[b], acc[b][mb]);
          acc[b][mb] = mma_bf16(vf, L[b], acc[b][mb]);
        }
      }
    }
  }
  // A operand of row block mb from raw V chunks in registers (row d = NM c + mb): slot pair
  // (2p, 2p+1) takes dim mb of keys vkey(2p), vkey(2p+1). Pure data movement.
  __device__ static inline u32x4 pack_v(const VRow (&r)[8], int mb) {
    const int w = mb >> 1;
    unsigned out[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const unsigned a = r[2 * p][w], b = r[2 * p + 1][w];
      out[p] = (mb & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    return u32x4{out[0], out[1], out[2], out[3]};
  }
  // A operand of row block mb straight from a row-major V sub-tile in LDS, for the head-dim
  // mapping d = 16 mb + c, with two transposing reads (ds_read_b64_tr_b16). In each 16-lane
  // group the read hands lane i element i % 4 of the 8-byte chunks named by lanes i / 4 + 4 k,
  // k = 0..3; so when lane j names dims [16 mb + 4 (j % 4), +4) of key KEY(j / 4), lane c
  // receives dim 16 mb + c of keys KEY(0..3). KEY(k) = 4 g + k gives slots 0..3 and
  // 16 + 4 g + k slots 4..7, the keys the score layout left in this lane group.
  // The same two transposing reads at a precomputed lane address p (the first 16 keys' row)
  // and p + gap (the row 16 keys later), for swizzled tile layouts.
  __device__ static inline u32x4 v_tr_at(const char* p, int gap) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + gap));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
  __device__ static inline u32x4 v_tr(const char* vt, int stride, int mb, int c, int g) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
    const int col = (16 * mb + 4 * (c & 3)) * 2;
    const char* r0 = vt + (4 * g + (c >> 2)) * stride + col;
    const char* r1 = r0 + 16 * stride;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)r0);
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)r1);
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    return u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
};

// fp32: QK^T in D/4 k-steps of v_mfma_f32_16x16x4_f32; lane (c, g) holds dim (D/4) g + s of
// k-step s. PV in 8 k-steps (kb, r): slot g is key 16 kb + 4 g + r, the lane's own score.
template <int D> struct Frag<float, D> {
  static constexpr int NKS = D / 4;
  static constexpr int NM = D / 16;
  static constexpr int ROWB = D * 4;
  using KOp = float;
  struct VRow { float v[NM]; };
  struct Q { float v[NKS]; };
  struct VRaw { VRow v[8]; };

  __device__ static inline int vkey(int i, int g) { return 16 * (i >> 2) + 4 * g + (i & 3); }
  __device__ static inline KOp k_op(const char* row, int st, int g) {
    return *(const float*)(row + (NKS * g + st) * 4);
  }
  __device__ static inline KOp zero_k() { return 0.f; }
  __device__ static inline VRow v_row(const char* row, int c) {
    VRow r;
    const f32x4* p = (const f32x4*)(row + NM * c * 4);
#pragma unroll
    for (int s = 0; s < NM / 4; ++s) {
      const f32x4 t = p[s];
      r.v[4 * s] = t[0]; r.v[4 * s + 1] = t[1]; r.v[4 * s + 2] = t[2]; r.v[4 * s + 3] = t[3];
    }
    return r;
  }
  // the same loads marked non-temporal (streaming: data read once, not kept in the caches)
  __device__ static inline KOp k_op_nt(const char* row, int st, int g) {
    return __builtin_nontemporal_load((const float*)(row + (NKS * g + st) * 4));
  }
  __device__ static inline VRow v_row_nt(const char* row, int c) {
    VRow r;
    const f32x4* p = (const f32x4*)(row + NM * c * 4);
#pragma unroll
    for (int s = 0; s < NM / 4; ++s) {
      const f32x4 t = __builtin_nontemporal_load(p + s);
      r.v[4 * s] = t[0]; r.v[4 * s + 1] = t[1]; r.v[4 * s + 2] = t[2]; r.v[4 * s + 3] = t[3];
    }
    return r;
  }
  __device__ static inline void store_k(char* row, int st, int g, KOp x) { *(float*)(row + (NKS * g + st) * 4) = x; }
  __device__ static inline void store_v(char* row, int c, const VRow& x) {
    f32x4* p = (f32x4*)(row + NM * c * 4);
#pragma unroll
    for (int s = 0; s < NM / 4; ++s) p[s] = f32x4{x.v[4 * s], x.v[4 * s + 1], x.v[4 * s + 2], x.v[4 * s + 3]};
  }
  __device__ static inline VRow zero_v() {
    VRow r;
#pragma unroll
    for (int m = 0; m < NM; ++m) r.v[m] = 0.f;
    return r;
  }
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
  template <int NB, bool PIPE = false, class KGet>
  __device__ static inline void qk(f32x4 (&s)[NB][2], KGet& getK, const Q (&q)[NB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        const float kf = getK(kb, st);
#pragma unroll
        for (int b = 0; b < NB; ++b) s[b][kb] = mma_f32(kf, q[b].v[st], s[b][kb]);
      }
    }
  }
  // getV(i) returns the lane's raw V chunk (NM floats, dims NM c .. NM c + NM) of key slot i.
  template <int NB, bool PIPE = false, class VGet>
  __device__ static inline void pv(f32x4 (&acc)[NB][NM], VGet& getV, const float (&p)[NB][2][4],
                                   float (&)[NB], const bool (&)[NB], bool, const u32x4 (&)[2]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const VRow row = getV(i);
#pragma unroll
      for (int mb = 0; mb < NM; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[b][mb] = mma_f32(row.v[mb], p[b][i >> 2][i & 3], acc[b][mb]);
    }
  }
};

// ------------------------------------------------------------------------------------------
// Softmax state of one query row (one lane group), in base-2 units: p = 2^(q.k c - m) with
// c = scale * log2(e); l = sum p; acc = sum p v. m is a reference maximum: it is set to the
// sub-tile row max at the start of a split and raised only when a later row max exceeds it
// by more than kLazy (so p <= 2^kLazy). The result is the same softmax; skipping most
// rescales removes the acc *= alpha multiplies from most sub-tiles. The decision depends on
// the row's own numbers only, so every route makes the same one.
// l is kept per lane: the sum of the weights the lane's PV products used (bf16 data: its P_hi
// and P_lo values, added by Frag::pv; fp32 data: its p values); the row's l is the sum of its
// four lanes' partials, taken once per split by row_l().
constexpr float kLazy = 8.0f;
// Precision of P in the bf16 PV product. P_hi = bf16(p) alone carries a relative error up to
// 2^-9 per key, which reaches the output in proportion to the key's share of the softmax: a
// few keys carrying most of the weight pass it on almost whole. The P_lo term (p - P_hi, a
// second bf16) is added for the keys of a lane when either holds:
//   * the row is at a position below kLoKeys (few keys, so every key's share is large);
//   * the row's split is peaked: from the sub-tile on where some lane of the row holds a
//     scaled score more than kGap (base-2 units) above the mean of the row's unmasked scaled
//     scores in the split's first sub-tile, to the end of the split. N(0,1)-like rows put
//     their largest scores about 3 above that mean and pass 7, about 4.9 standard deviations,
//     in about one split in 3000; sharper softmaxes pass it within a sub-tile or two, and so
//     does a lone outlier key.
// Each decision depends only on the row's own scores and position, so every route takes the
// same one; lanes without P_lo add exact zeros.
constexpr int kLoKeys = 1024;
constexpr float kGap = 7.0f;
__device__ __forceinline__ bool needs_lo(int pos) { return pos >= 0 && pos < kLoKeys; }

template <int D> struct RowState {
  static constexpr int NM = D / 16;
  float m, l;
  float gate;  // raw score of the peaked-split test: (mean of the split's first sub-tile's
               // scaled scores + kGap) / cscale (NaN when that sub-tile has no unmasked key)
  bool lo;     // the split has turned out peaked: P_lo for its keys from then on
  f32x4 acc[NM];
};
template <int D> __device__ __forceinline__ float row_l(const RowState<D>& st) { return xor_sum(st.l); }

__device__ __forceinline__ bool wave_any(bool v) { return __builtin_amdgcn_ballot_w64(v) != 0; }

// One 32-key sub-tile of NB column blocks that share the K/V operands.
//   getK(kb, s)   -> K operand of key block kb, k-step s
//   getV(x)       -> PV A operand (bf16: of row block x; fp32: raw V chunk of key slot x)
//   pos[b]        -> this lane's row position in block b
//   first: first sub-tile of the split (state reset, not rescaled)
//   mask:  some key of the sub-tile may lie after some row's position (wave-uniform)
//   lo_pos[b]: needs_lo(pos[b]); lo_pos_w: some lane of the wave has it (wave-uniform); both
//          depend on the positions only, so callers compute them once
//   lo_wave: wave-uniform, nonzero when some row of the wave has its split's peaked flag set
//          (kept by the caller from one sub-tile of the split to the next; reset here at the
//          split's first sub-tile)
//   A row with pos < key0 (all its keys masked) takes p = 0 everywhere, which leaves its state
//   bitwise as it was; at a split start it gets the empty state (m = -FLT_MAX, l = 0,
//   acc = 0), which the ascending fold leaves bitwise unchanged (a = 1, b = 0).
//   PIPE:  operand reads are issued ahead of the MFMAs that use them (LDS operands): K one
//          k-step ahead, V two row blocks ahead
template <typename E, int D, int NB, bool PIPE = false, class KGet, class VGet>
__device__ __forceinline__ void subtile_step(RowState<D>* st, const typename Frag<E, D>::Q* q,
                                             const int* pos, KGet&& getK, VGet&& getV,
                                             float cscale, int key0, int g, bool first,
                                             bool mask, const bool (&lo_pos)[NB], bool lo_pos_w,
                                             int& lo_wave) {
  using F = Frag<E, D>;
  constexpr int NM = D / 16;
  typename F::Q qv[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) qv[b] = q[b];
  f32x4 s[NB][2];
  F::template qk<NB, PIPE>(s, getK, qv);
  // the first PV operands (bf16 with LDS operands), read while the softmax runs
  constexpr int NPRE = 2;
  u32x4 vpre[NPRE];
#pragma unroll
  for (int i = 0; i < NPRE; ++i) vpre[i] = u32x4{0, 0, 0, 0};
  if constexpr (PIPE) {
#pragma unroll
    for (int i = 0; i < NPRE; ++i) vpre[i] = getV(i);
    __builtin_amdgcn_sched_barrier(0);
  }
  float p[NB][2][4];
  float x[NB][2][4], mxl[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) x[b][kb][r] = s[b][kb][r];
    if (mask) {
      // key key0 + 16 kb + 4 g + r is visible to the row iff 16 kb + r <= pos - key0 - 4 g
      const int lim = pos[b] - key0 - 4 * g;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) x[b][kb][r] = (16 * kb + r <= lim) ? x[b][kb][r] : -__builtin_inff();
    }
    mxl[b] = vmax(vmax3(x[b][0][0], x[b][0][1], x[b][0][2]),
                  vmax3(x[b][0][3], x[b][1][0], vmax3(x[b][1][1], x[b][1][2], x[b][1][3])));
  }
  float mnew[NB], alpha[NB], lnew[NB];
  constexpr bool BF = std::is_same<E, __bf16>::value;
  // The common sub-tile of a long prefill: not the split's first, no masked key, no row that
  // needs P_lo, and no lane above its row's gate. The general code then keeps every reference
  // (alpha = 1, l carried as it is, no rescale) and the peaked flags; this branch is that code
  // with those values put in, so it gives the same bits without the decision chain.
  bool fast = false;
  if constexpr (PIPE) {
    if (!first && !mask && !lo_pos_w && lo_wave == 0) {
      unsigned long long hit = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) hit |= __builtin_amdgcn_ballot_w64(mxl[b] > st[b].gate);
      fast = hit == 0;
    }
  }
  if (fast) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      mnew[b] = st[b].m;
      const float nm = -st[b].m;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[b][kb][r] = ex2(__builtin_fmaf(x[b][kb][r], cscale, nm));
      if constexpr (BF) {
        lnew[b] = st[b].l;   // the P words are added by pv()
      } else {
        const float rs = ((p[b][0][0] + p[b][0][1]) + (p[b][0][2] + p[b][0][3])) +
                         ((p[b][1][0] + p[b][1][1]) + (p[b][1][2] + p[b][1][3]));
        lnew[b] = __builtin_fmaf(st[b].l, 1.0f, rs);
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      mnew[b] = st[b].m;
      alpha[b] = 1.0f;
    }
    bool rescale = false;
    // Past the split's first sub-tile, a sub-tile none of whose lanes holds a raw score above
    // its row's gate needs no decision: the gate is at least one base-2 unit below m + kLazy
    // once scaled (m is at least the first sub-tile's max, so at least its mean), so no row
    // raises its reference, and the peaked flag stays as it is. One compare per block.
    unsigned long long gate_hit = 0;
    if (!first) {
#pragma unroll
      for (int b = 0; b < NB; ++b) gate_hit |= __builtin_amdgcn_ballot_w64(mxl[b] > st[b].gate);
    }
    if (first || gate_hit != 0) {
      // A row raises its reference only if some lane of it holds a scaled score above
      // m + kLazy (the scaled row max is the max of the lanes' scaled maxima: rounding is
      // monotonic), so the row max butterfly runs only at a split start or when some lane of the
      // wave needs it.
      bool full = first;
      if (!first) {
        unsigned long long up = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) up |= __builtin_amdgcn_ballot_w64(mxl[b] * cscale > st[b].m + kLazy);
        full = up != 0;
      }
      if (full) {
        unsigned long long need_any = 0;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float rm = xor_max(mxl[b]);
          const float mt = rm * cscale;
          if (first) {
            // an all-masked row (a prefill row below the split's first key) takes the reference
            // -FLT_MAX, so its p = 2^-inf = 0 with a finite offset
            mnew[b] = mt > -3.40282347e38f ? mt : -3.40282347e38f;
            // gate of the peaked-split test: (mean of the row's unmasked scaled scores + kGap) /
            // cscale: the lane's scores summed in a fixed order, the row sum by the xor butterfly
            // (every lane of the row gets the same bits), divided by the unmasked count
            // min(32, pos - key0 + 1) through v_rcp_f32; an all-masked row gets 0 * inf = NaN,
            // which never tests true
            float sum = 0.f, rcnt = 1.0f / kSubTile;
            if (mask) {
#pragma unroll
              for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sum = sum + (x[b][kb][r] > -__builtin_inff() ? x[b][kb][r] : 0.f);
              rcnt = __builtin_amdgcn_rcpf((float)min(max(pos[b] - key0 + 1, 0), kSubTile));
            } else {
#pragma unroll
              for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) sum = sum + x[b][kb][r];
            }
            sum = xor_sum(sum);
            st[b].gate = (sum * cscale * rcnt + kGap) * __builtin_amdgcn_rcpf(cscale);
            st[b].lo = false;
          } else {
            const bool need = mt > st[b].m + kLazy;
            if (need) {
              mnew[b] = mt;
              alpha[b] = ex2(st[b].m - mt);
            }
            need_any |= __builtin_amdgcn_ballot_w64(need);
          }
        }
        rescale = !first && need_any != 0;
      }
      // the split's peaked flag (per row, sticky): a ballot of the lanes above their row's gate,
      // read out for the lanes c, c + 16, c + 32, c + 48 of each row
      const int col = (int)(threadIdx.x & 15);
      unsigned long long any_lo = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const unsigned long long up = __builtin_amdgcn_ballot_w64(mxl[b] > st[b].gate);
        st[b].lo = st[b].lo || ((up >> col) & 0x0001000100010001ull) != 0;
        any_lo |= __builtin_amdgcn_ballot_w64(st[b].lo);
      }
      lo_wave = any_lo != 0;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float nm = -mnew[b];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[b][kb][r] = ex2(__builtin_fmaf(x[b][kb][r], cscale, nm));
      if constexpr (BF) {
        // the part of l carried into the sub-tile (l alpha is l itself where the reference
        // stays); pv() adds the P words
        lnew[b] = first ? 0.f : st[b].l * alpha[b];
      } else {
        const float rs = ((p[b][0][0] + p[b][0][1]) + (p[b][0][2] + p[b][0][3])) +
                         ((p[b][1][0] + p[b][1][1]) + (p[b][1][2] + p[b][1][3]));
        lnew[b] = first ? rs : __builtin_fmaf(st[b].l, alpha[b], rs);
      }
    }
    if (first) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mb = 0; mb < NM; ++mb) st[b].acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (rescale) {
      // alpha == 1 exactly for rows that kept their reference, so x * alpha == x
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mb = 0; mb < NM; ++mb) st[b].acc[mb] = st[b].acc[mb] * alpha[b];
    }
  }
  // P_lo choice of this lane's keys: the row's position or the split's peaked flag
  bool lo_row[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) lo_row[b] = lo_pos[b] || st[b].lo;
  const bool lo_any = lo_pos_w || lo_wave != 0;
  f32x4 accl[NB][NM];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) accl[b][mb] = st[b].acc[mb];
  F::template pv<NB, PIPE>(accl, getV, p, lnew, lo_row, lo_any, vpre);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    st[b].m = mnew[b];
    st[b].l = lnew[b];
#pragma unroll
    for (int mb = 0; mb < NM; ++mb) st[b].acc[mb] = accl[b][mb];
  }
}

// Ascending fold of split j's state into the row state (the same function the combine kernel
// applies element by element), with a lazy row reference like the one inside a split: M is
// raised to the split's m only when m exceeds it by more than kLazy, and then a = 2^(M - m),
// b = 1; otherwise M stays, a = 1 and b = 2^(m - M) <= 2^kLazy. L = l b + L a and
// A = acc b + A a, each one fma with the rounded product of the row state as addend (so A can
// be updated in place). Where a = 1 that product is the row state itself, so a caller may skip
// the multiply when no lane raises (fold_raises) and still get the same bits. The row state
// starts at (M, L, A) = (-inf, 0, 0), so split 0 raises (a = 0, b = 1) and copies its state
// exactly (x 1 + 0 = x for the never negative-zero partials) with no special case; an empty
// split (m = -FLT_MAX, l = 0, acc = 0) after a finite M gives b = 0 and leaves the row state as
// it was; a NaN m or M gives b = NaN, so the row comes out NaN.
__device__ __forceinline__ bool fold_raises(float M, float m) { return m > M + kLazy; }
__device__ __forceinline__ void fold_scalars(float& M, float& L, float m, float l, float& a, float& b) {
  const bool up = fold_raises(M, m);
  const float e = ex2(up ? M - m : m - M);
  a = up ? e : 1.0f;
  b = up ? 1.0f : e;
  L = __builtin_fmaf(l, b, L * a);
  M = up ? m : M;
}
__device__ __forceinline__ float fold_elem(float A, float acc, float a, float b) {
  return __builtin_fmaf(acc, b, A * a);
}

}  // namespace bi
