// bi_gemm.hip — batch-invariant GEMM C = A W^T (gfx950): output tiles of 256 x 256, 128 x 128
// or 64 x 64 (or 32 x 32 per wave for few rows and long K), the whole of K inside one workgroup
// in ascending order, MFMA 32x32x16 bf16.
//
// The matmul is made batch invariant by a fixed tile configuration with no Split-K (xitu-tech.com
// report, section 构建确定性解决方案, matrix multiplication item): the output is cut into 2-D tiles
// and each core finishes its dot products itself (neican.ai insight page, section
// 技术原理与创新点解析, matmul item). Here a workgroup owns one tile of C and reduces all of K
// for it; the order of a C element's products (16-wide MFMA k-substeps, ascending, each into the
// one fp32 accumulator) is the same for every M, every tile shape and every tile position.
//
// Data path: A and W tiles go HBM -> LDS by buffer loads to LDS (buffer_load_dwordx4 ... lds: no
// register staging; a scalar resource per operand tile and 32-bit lane offsets; the compiler
// counts them on the vector-memory counter only, so the operand reads wait for just what they
// need, where a global_load_lds would turn each wait into a wait for every LDS read in flight:
// 12-18% faster here), a ring of 2 to 4 stages (each a separate LDS variable) filled up to
// stages - 1 K steps ahead, one barrier per K step that waits only for the oldest step. LDS rows
// are BK bf16; a row's 16-byte chunks are permuted by phys_chunk so that the operand reads (32
// rows at one chunk) hit distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/bi_gemm.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kKAlign = 64;                      // K must be a multiple of this
// s_waitcnt operands: vmcnt <= n only (expcnt and lgkmcnt at their maximum), and vmcnt <= n
// with lgkmcnt = 0 (every LDS read of the wave returned)
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int wait_vm_lds0(int n) { return 0x0070 | (n & 15) | ((n >> 4) << 14); }
// A wave computes TM x TN MFMA tiles of 32 x 32 (rows x columns of C); NWV waves (4 or 8) form a
// 2 x NWV / 2 grid, so the workgroup tile is BM x BN = 64 TM x 16 TN NWV, staged BK columns of K
// at a time. Neither the tile shape, the wave count nor BK changes any element's order of
// products (16-wide MFMA k-substeps, ascending).
template <int TM, int TN, int BK_, int NWV_ = 4> struct GemmTile {
  static constexpr int BK = BK_, CPR = BK / 8;   // 16-byte chunks per LDS row
  static constexpr int NWV = NWV_, NT = 64 * NWV, WGN = NWV / 2;
  static constexpr int BM = 64 * TM, BN = 32 * TN * WGN;
  static constexpr int A_BYTES = BM * BK * 2, W_BYTES = BN * BK * 2;
  static constexpr int A_ROUNDS = BM * CPR / NT, W_ROUNDS = BN * CPR / NT;
  static_assert(A_ROUNDS * NT == BM * CPR && W_ROUNDS * NT == BN * CPR, "tile vs threads");
};

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in that order
template <int N, int J = 0, class F> __device__ __forceinline__ void for_stages(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>{});
    for_stages<N, J + 1>(f);
  }
}

// Chunk c of LDS row R is stored at chunk phys_chunk(c, R): the 16 rows that one pass of a
// 16-byte operand read touches (one chunk each) then fall on 16 distinct 16-byte bank groups.
template <int CPR> __device__ __forceinline__ int phys_chunk(int c, int row) {
  if constexpr (CPR == 8) return c ^ ((row >> 1) & 7);
  else return c ^ ((row >> 2) & 3);
}

template <bool OUT_BF16, int TM, int TN, int BK, int NS, int NWV, int MINB>
__global__ __launch_bounds__(64 * NWV, MINB) void gemm_kernel(const char* A, const char* W, char* C, int M,
                                                              int N, int K) {
  using T = GemmTile<TM, TN, BK, NWV>;
  constexpr int NT = T::NT, WGN = T::WGN;
  constexpr int BM = T::BM, BN = T::BN, CPR = T::CPR, KS = BK / 16;
  // NS stages: K step kt lives in stage kt % NS. Each stage is a variable of its own, so the
  // compiler can tell that the reads of one stage do not wait for the transfers into another.
  static_assert(NS >= 2 && NS <= 8, "stages");
#define BI_GEMM_STAGE(i)                                                                     \
  __shared__ __attribute__((aligned(16))) char sa##i[NS > i ? T::A_BYTES : 16];               \
  __shared__ __attribute__((aligned(16))) char sw##i[NS > i ? T::W_BYTES : 16];
  BI_GEMM_STAGE(0) BI_GEMM_STAGE(1) BI_GEMM_STAGE(2) BI_GEMM_STAGE(3)
  BI_GEMM_STAGE(4) BI_GEMM_STAGE(5) BI_GEMM_STAGE(6) BI_GEMM_STAGE(7)
#undef BI_GEMM_STAGE
  // stage J's buffers, named directly (no pointer table, so every access keeps its LDS address
  // space and its variable)
  auto stage_a = [&](auto J) __attribute__((always_inline)) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sa0; else if constexpr (j == 1) return sa1;
    else if constexpr (j == 2) return sa2; else if constexpr (j == 3) return sa3;
    else if constexpr (j == 4) return sa4; else if constexpr (j == 5) return sa5;
    else if constexpr (j == 6) return sa6; else return sa7;
  };
  auto stage_w = [&](auto J) __attribute__((always_inline)) -> char* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sw0; else if constexpr (j == 1) return sw1;
    else if constexpr (j == 2) return sw2; else if constexpr (j == 3) return sw3;
    else if constexpr (j == 4) return sw4; else if constexpr (j == 5) return sw5;
    else if constexpr (j == 6) return sw6; else return sw7;
  };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ntn = N / BN;
  const int tm = (int)blockIdx.x / ntn, tn = (int)blockIdx.x - tm * ntn;
  const int m0 = tm * BM, n0 = tn * BN;
  const size_t rowb = (size_t)K * 2;               // bytes per row of A and W

  // DMA: slot p = NT t + 64 wave + lane of a tile is LDS row p / CPR, physical chunk p % CPR,
  // which holds the logical chunk that phys_chunk maps there (phys_chunk is an involution).
  // Rows of A past M read row M - 1 (their outputs are not written).
  unsigned a_vo[T::A_ROUNDS], w_vo[T::W_ROUNDS];
#pragma unroll
  for (int t = 0; t < T::A_ROUNDS; ++t) {
    const int p = NT * t + 64 * wave + lane, R = p / CPR;
    a_vo[t] = (unsigned)((min(m0 + R, M - 1) - m0) * rowb) + phys_chunk<CPR>(p % CPR, R) * 16;
  }
#pragma unroll
  for (int t = 0; t < T::W_ROUNDS; ++t) {
    const int p = NT * t + 64 * wave + lane, R = p / CPR;
    w_vo[t] = (unsigned)(R * rowb) + phys_chunk<CPR>(p % CPR, R) * 16;
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // (the buffer builtins exist only in the device pass; the host pass never runs this body)
  const char* abase = A + (size_t)m0 * rowb;
  const char* wbase = W + (size_t)n0 * rowb;
  auto dma = [&](int kt, char* da, char* dw) __attribute__((always_inline)) {
    const unsigned kb = (unsigned)kt * BK * 2;
#if defined(__HIP_DEVICE_COMPILE__)
    const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(abase), (short)0, 0x7fffffff, 0x00020000);
    const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wbase), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int t = 0; t < T::A_ROUNDS; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)&da[(NT * t + 64 * wave) * 16], 16, a_vo[t] + kb, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < T::W_ROUNDS; ++t)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_ptr)&dw[(NT * t + 64 * wave) * 16], 16, w_vo[t] + kb, 0, 0, 0);
#endif
  };

  // operand reads: A rows (BM / 2) wm + 32 i + lane % 32, W rows (BN / WGN) wn + 32 j + lane % 32,
  // logical chunk 2 ks + lane / 32 (k = 16 ks + 8 (lane / 32) .. + 7)
  const int wm = wave & 1, wn = wave >> 1;
  unsigned rd_a[TM][KS], rd_w[TN][KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int c = 2 * ks + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ra = (BM / 2) * wm + 32 * i + (lane & 31);
      rd_a[i][ks] = (unsigned)(ra * BK * 2 + phys_chunk<CPR>(c, ra) * 16);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int rw = (BN / WGN) * wn + 32 * j + (lane & 31);
      rd_w[j][ks] = (unsigned)(rw * BK * 2 + phys_chunk<CPR>(c, rw) * 16);
    }
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](const char* sa, const char* sw) __attribute__((always_inline)) {
    u32x4 a[TM], w[TN], an[TM], wn_[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *(const u32x4*)&sa[rd_a[i][0]];
#pragma unroll
    for (int j = 0; j < TN; ++j) w[j] = *(const u32x4*)&sw[rd_w[j][0]];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < TM; ++i) an[i] = *(const u32x4*)&sa[rd_a[i][ks + 1]];
#pragma unroll
        for (int j = 0; j < TN; ++j) wn_[j] = *(const u32x4*)&sw[rd_w[j][ks + 1]];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                              __builtin_bit_cast(bf16x8, w[j]), acc[i][j], 0, 0, 0);
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < TM; ++i) a[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) w[j] = wn_[j];
      }
    }
  };

  // Step kt: wait for this wave's transfers of step kt (the later NS - 2 steps' may still be in
  // flight), barrier (every wave's transfers of step kt have landed, and every wave is done with
  // step kt - 1), refill the stage of step kt - 1 with step kt + NS - 1, compute step kt.
  // Transfers past the last step re-load it into stages that are not read again, so every step
  // issues the same number of transfers and the wait count is the same constant throughout.
  constexpr int R = T::A_ROUNDS + T::W_ROUNDS;   // transfers per step per wave
  const int KT = K / BK;
  for_stages<NS - 1>([&](auto J) __attribute__((always_inline)) {
    dma(min((int)decltype(J)::value, KT - 1), stage_a(J), stage_w(J));
  });
  auto body = [&](int kt, auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    using Jn = std::integral_constant<int, (j + NS - 1) % NS>;
    // A plain barrier, not __syncthreads(): its release fence would wait for every transfer in
    // flight. None is needed here: LDS has no cache, a wave's transfers are in LDS once its
    // vmcnt has dropped, and lgkmcnt = 0 means every LDS read of the wave (those of the stage
    // refilled below included) has returned before it reaches the barrier. The empty asm
    // keeps the compiler from moving memory accesses across the barrier.
    __builtin_amdgcn_s_waitcnt(wait_vm_lds0((NS - 2) * R));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    dma(min(kt + NS - 1, KT - 1), stage_a(Jn{}), stage_w(Jn{}));
    compute(stage_a(J), stage_w(J));
  };
  // whole rounds of NS steps (one loop exit, so the accumulators stay in place), then the rest
  const int rounds = KT / NS, rest = KT - rounds * NS;
  for (int r = 0; r < rounds; ++r)
    for_stages<NS>([&](auto J) __attribute__((always_inline)) { body(r * NS + decltype(J)::value, J); });
  for_stages<NS>([&](auto J) __attribute__((always_inline)) {
    if (decltype(J)::value < rest) body(rounds * NS + decltype(J)::value, J);
  });
  // the transfers past the last step must land before the workgroup's LDS can be handed on
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // epilogue: element e of acc[i][j] is C row (BM / 2) wm + 32 i + 8 (e / 4) + 4 (lane / 32) +
  // e % 4, column (BN / WGN) wn + 32 j + lane % 32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + (BM / 2) * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= M) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int col = n0 + (BN / WGN) * wn + 32 * j + (lane & 31);
        const float v = acc[i][j][e];
        if constexpr (OUT_BF16) ((__bf16*)C)[(size_t)r * N + col] = (__bf16)v;
        else ((float*)C)[(size_t)r * N + col] = v;
      }
    }
}

// Skinny products (few rows of A): one wave per workgroup owns a 32 TM x 32 tile of C and loads
// its A and W operands straight into registers, P 16-wide k-substeps ahead of the MFMA that uses
// them (a ring of P operand sets, so that enough bytes of W are in flight with only N / 32 waves);
// no LDS, no barrier. Lane l loads, for k-substep s, the 16 bytes k = 16 s + 8 (l / 32) .. + 7 of
// A row 32 i + l % 32 (rows past M read row M - 1) and of W row l % 32 of the tile: the operands,
// MFMA and accumulation order of the tiled kernel above, so every element has the same bits.
template <bool OUT_BF16, int TM, int P>
__global__ __launch_bounds__(64) void gemm_skinny_kernel(const char* A, const char* W, char* C, int M, int N,
                                                         int K) {
  const int lane = threadIdx.x;
  const int n0 = (int)blockIdx.x * 32, m0 = (int)blockIdx.y * 32 * TM;
  const size_t rowb = (size_t)K * 2;
  const int ks_total = K / 16;
  const char* wrow = W + (size_t)(n0 + (lane & 31)) * rowb + (lane >> 5) * 16;
  const char* arow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = A + (size_t)min(m0 + 32 * i + (lane & 31), M - 1) * rowb + (lane >> 5) * 16;
  u32x4 wr[P], ar[P][TM];
  // substep s lives in slot s % P; loads past the last substep re-read it (never used)
  auto load = [&](int slot, int s) __attribute__((always_inline)) {
    const size_t off = (size_t)min(s, ks_total - 1) * 32;
    wr[slot] = *(const u32x4*)(wrow + off);
#pragma unroll
    for (int i = 0; i < TM; ++i) ar[slot][i] = *(const u32x4*)(arow[i] + off);
  };
#pragma unroll
  for (int p = 0; p < P; ++p) load(p, p);
  f32x16 acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  auto step = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ar[slot][i]),
                                                       __builtin_bit_cast(bf16x8, wr[slot]), acc[i], 0, 0, 0);
  };
  // whole rounds of P substeps (a branch-free body, so the loads of one round stay in flight
  // across the loop edge), then the rem < P substeps left, from the ring as it stands
  const int rounds = ks_total / P, rem = ks_total - rounds * P;
  for (int r = 1; r <= rounds; ++r) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      step(p);
      load(p, r * P + p);
      __builtin_amdgcn_sched_barrier(0);   // keep each refill right behind the MFMA it follows
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p < rem) step(p);
  // element e of acc[i]: C row m0 + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4, column n0 + lane % 32
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= M) continue;
      const int col = n0 + (lane & 31);
      if constexpr (OUT_BF16) ((__bf16*)C)[(size_t)r * N + col] = (__bf16)acc[i][e];
      else ((float*)C)[(size_t)r * N + col] = acc[i][e];
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Products with at most kSkinnyMaxM rows and a K of at least kSkinnyMinK take the skinny kernel
// (one 32-row tile, a ring of 24 substeps): there it has twice the workgroups of the 64 x 64
// tiles (N / 32) and streams W 1.0-1.4x faster than they do on MI355X (M = 1 to 16, K = 8192
// and 14336); at K = 4096 the staged 64 x 64 tiles are as fast or faster.
constexpr int kSkinnyMaxM = 16, kSkinnyMinK = 8192;

template <int TM, int P>
int launch_skinny(const void* a, const void* w, void* c, int m, int n, int k, int c_dtype, hipStream_t stream) {
  const dim3 grid((unsigned)(n / 32), (unsigned)((m + 32 * TM - 1) / (32 * TM)));
  if (c_dtype == 1)
    hipLaunchKernelGGL((gemm_skinny_kernel<true, TM, P>), grid, dim3(64), 0, stream, (const char*)a,
                       (const char*)w, (char*)c, m, n, k);
  else
    hipLaunchKernelGGL((gemm_skinny_kernel<false, TM, P>), grid, dim3(64), 0, stream, (const char*)a,
                       (const char*)w, (char*)c, m, n, k);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Large products take 256 x 256 workgroup tiles (one workgroup of 8 waves per CU, 128 x 64 per
// wave, two waves per SIMD so that one's barrier and transfer waits overlap the other's MFMAs:
// 6-10% faster than 4 waves of 128 x 128 on MI355X; half the fabric traffic per flop of the
// 128 x 128 tile, which keeps 4 waves: 8 measured 2-3% slower there); products
// with fewer than kBigTilesMin such tiles take 128 x 128 tiles, so the grid still fills the chip
// (160 rather than 256, one per CU: 7-15% faster on MI355X for shapes with 160 to 255 large tiles,
// e.g. 1536 x 8192, 3072 x 4096, whose 128 x 128 tiles would run a second, partial round).
// Both walk every element's K in the same 16-wide MFMA steps (as do the 64 x 64 tiles and the
// skinny kernel), so their bits are identical and the choice, which depends on M, cannot make a
// row's result depend on M.
constexpr int kBigTilesMin = 160;

// LDS stages per tile shape (64-wide K steps): 256 x 256 tiles 2 (128 KB), 128 x 128 tiles 2
// (64 KB, two workgroups per CU), 64 x 64 tiles 4 (64 KB): measured on MI355X, more stages (or
// 32-wide K steps with more stages) gained nothing for the larger tiles, and cut the 64 x 64
// tiles' time by half or more.
// Products with fewer than kMidTilesMax tiles of 128 x 128 (M from 65 to a few hundred) take
// 64 x 64 tiles (32 x 32 per wave): four times the workgroups; 20-35% faster there on MI355X.
constexpr int kMidTilesMax = 256;

template <int TM, int TN, int BK, int NS, int NWV = 4>
int launch_gemm(const void* a, const void* w, void* c, int m, int n, int k, int c_dtype, hipStream_t stream) {
  using T = GemmTile<TM, TN, BK, NWV>;
  constexpr int MINB = (NS * (T::A_BYTES + T::W_BYTES) <= 80 * 1024) ? 2 : 1;
  if (n % T::BN) return 2;
  const int64_t tiles = (((int64_t)m + T::BM - 1) / T::BM) * (n / T::BN);
  if (tiles > 0x7fffffff) return 2;
  if (c_dtype == 1)
    hipLaunchKernelGGL((gemm_kernel<true, TM, TN, BK, NS, NWV, MINB>), dim3((unsigned)tiles), dim3(T::NT), 0, stream,
                       (const char*)a, (const char*)w, (char*)c, m, n, k);
  else
    hipLaunchKernelGGL((gemm_kernel<false, TM, TN, BK, NS, NWV, MINB>), dim3((unsigned)tiles), dim3(T::NT), 0, stream,
                       (const char*)a, (const char*)w, (char*)c, m, n, k);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace

extern "C" int bi_gemm(const void* a, const void* w, void* c, int32_t m, int32_t n, int32_t k,
                       int32_t c_dtype, hipStream_t stream) {
  if (c_dtype != 0 && c_dtype != 1) return 1;
  if (m < 0 || n <= 0 || k <= 0) return 1;
  if (n % 128 || k % kKAlign) return 2;
  if ((int64_t)k * 2 * 256 >= ((int64_t)1 << 31)) return 2;   // 32-bit lane offsets inside a tile
  if (m == 0) return 0;
  if (!a || !w || !c || !aligned16(a) || !aligned16(w) || !aligned16(c)) return 1;
  if (m <= kSkinnyMaxM && k >= kSkinnyMinK) return launch_skinny<1, 24>(a, w, c, m, n, k, c_dtype, stream);
  const int64_t big_tiles = (((int64_t)m + 255) / 256) * (n / 256);
  if (n % 256 == 0 && big_tiles >= kBigTilesMin) return launch_gemm<4, 2, 64, 2, 8>(a, w, c, m, n, k, c_dtype, stream);
  const int64_t tiles128 = (((int64_t)m + 127) / 128) * (n / 128);
  if (tiles128 < kMidTilesMax) return launch_gemm<1, 1, 64, 4>(a, w, c, m, n, k, c_dtype, stream);
  return launch_gemm<2, 2, 64, 2, 4>(a, w, c, m, n, k, c_dtype, stream);
}
