// bi_gemm.hip — batch-invariant GEMM C = A W^T (gfx950): fixed 128 x 128 output tiles, the whole
// of K inside one workgroup in ascending order, MFMA 32x32x16 bf16.
//
// The matmul is made batch invariant by a fixed tile configuration with no Split-K (xitu-tech.com
// report, section 构建确定性解决方案, matrix multiplication item): the output is cut into 2-D tiles
// and each core finishes its dot products itself (neican.ai insight page, section
// 技术原理与创新点解析, matmul item). Here a workgroup owns one 128 x 128 tile of C and reduces
// all of K for it; the order of a C element's products (64-wide K steps ascending, 16-wide MFMA
// k-substeps ascending inside a step) is the same for every M and every tile position.
//
// Data path: A and W tiles go HBM -> LDS by global_load_lds_dwordx4 (no register staging), two
// buffers as separate LDS variables, one barrier per K step. LDS rows are 64 bf16 (128 bytes);
// the 16-byte chunk c of row R sits at chunk c ^ ((R >> 1) & 7), so the operand reads (32 rows
// at one chunk, eight lanes at a time) hit distinct banks.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bi_gemm.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int BM = 128, BN = 128, BK = 64;      // workgroup tile and K step
constexpr int kThreadsG = 256;                   // 4 waves: 2 x 2 of 64 x 64
constexpr int TILE_BYTES = BM * BK * 2;          // 16 KB per operand tile
constexpr int kWaitVm0 = 0x0F70;                 // s_waitcnt vmcnt(0)

__device__ __forceinline__ int phys_chunk(int c, int row) { return c ^ ((row >> 1) & 7); }

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreadsG, 2) void gemm_kernel(const char* A, const char* W, char* C, int M,
                                                           int N, int K) {
  __shared__ __attribute__((aligned(16))) char lds0[2][TILE_BYTES];   // [A, W], even K steps
  __shared__ __attribute__((aligned(16))) char lds1[2][TILE_BYTES];   // [A, W], odd K steps
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int ntn = N / BN;
  const int tm = (int)blockIdx.x / ntn, tn = (int)blockIdx.x - tm * ntn;
  const int m0 = tm * BM, n0 = tn * BN;
  const size_t rowb = (size_t)K * 2;               // bytes per row of A and W

  // DMA: slot p = 256 t + 64 wave + lane of a tile (t = 0..3) is LDS row p / 8, physical chunk
  // p % 8, which holds logical chunk (p % 8) ^ ((row >> 1) & 7) of that row. Rows of A past M
  // read row M - 1 (their outputs are not written).
  const char* a_row[4];
  const char* w_row[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int p = 256 * t + 64 * wave + lane, R = p >> 3;
    const size_t coff = (size_t)phys_chunk(p & 7, R) * 16;
    a_row[t] = A + (size_t)min(m0 + R, M - 1) * rowb + coff;
    w_row[t] = W + (size_t)(n0 + R) * rowb + coff;
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  auto dma = [&](int kt, char (&dst)[2][TILE_BYTES]) __attribute__((always_inline)) {
    const size_t kb = (size_t)kt * BK * 2;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      __builtin_amdgcn_global_load_lds((const void*)(a_row[t] + kb), (lds_ptr)&dst[0][(256 * t + 64 * wave) * 16], 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(w_row[t] + kb), (lds_ptr)&dst[1][(256 * t + 64 * wave) * 16], 16, 0, 0);
    }
  };

  // operand reads: A rows wm 64 + 32 rb + lane % 32, W rows wn 64 + 32 cb + lane % 32, logical
  // chunk 2 ks + lane / 32 (k = 16 ks + 8 (lane / 32) .. + 7)
  const int wm = wave & 1, wn = wave >> 1;
  unsigned rd_a[2][4], rd_w[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ra = 64 * wm + 32 * i + (lane & 31), rw = 64 * wn + 32 * i + (lane & 31);
      const int c = 2 * ks + (lane >> 5);
      rd_a[i][ks] = (unsigned)(ra * 128 + phys_chunk(c, ra) * 16);
      rd_w[i][ks] = (unsigned)(rw * 128 + phys_chunk(c, rw) * 16);
    }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute = [&](char (&src)[2][TILE_BYTES]) __attribute__((always_inline)) {
    u32x4 a[2], w[2], an[2], wn_[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *(const u32x4*)&src[0][rd_a[i][0]];
      w[i] = *(const u32x4*)&src[1][rd_w[i][0]];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          an[i] = *(const u32x4*)&src[0][rd_a[i][ks + 1]];
          wn_[i] = *(const u32x4*)&src[1][rd_w[i][ks + 1]];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                              __builtin_bit_cast(bf16x8, w[j]), acc[i][j], 0, 0, 0);
      if (ks + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          a[i] = an[i];
          w[i] = wn_[i];
        }
      }
    }
  };

  const int KT = K / BK;
  dma(0, lds0);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  for (int kt = 0; kt < KT; kt += 2) {
    if (kt + 1 < KT) dma(kt + 1, lds1);
    compute(lds0);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    if (kt + 1 >= KT) break;
    if (kt + 2 < KT) dma(kt + 2, lds0);
    compute(lds1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  }

  // epilogue: element e of acc[i][j] is C row 64 wm + 32 i + 8 (e / 4) + 4 (lane / 32) + e % 4,
  // column 64 wn + 32 j + lane % 32
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + 64 * wm + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (r >= M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + (lane & 31);
        const float v = acc[i][j][e];
        if constexpr (OUT_BF16) ((__bf16*)C)[(size_t)r * N + col] = (__bf16)v;
        else ((float*)C)[(size_t)r * N + col] = v;
      }
    }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int bi_gemm(const void* a, const void* w, void* c, int32_t m, int32_t n, int32_t k,
                       int32_t c_dtype, hipStream_t stream) {
  if (c_dtype != 0 && c_dtype != 1) return 1;
  if (m < 0 || n <= 0 || k <= 0) return 1;
  if (n % BN || k % BK) return 2;
  if (m == 0) return 0;
  if (!a || !w || !c || !aligned16(a) || !aligned16(w) || !aligned16(c)) return 1;
  const int64_t tiles = (((int64_t)m + BM - 1) / BM) * (n / BN);
  if (tiles > 0x7fffffff) return 2;
  if (c_dtype == 1)
    hipLaunchKernelGGL(gemm_kernel<true>, dim3((unsigned)tiles), dim3(kThreadsG), 0, stream,
                       (const char*)a, (const char*)w, (char*)c, m, n, k);
  else
    hipLaunchKernelGGL(gemm_kernel<false>, dim3((unsigned)tiles), dim3(kThreadsG), 0, stream,
                       (const char*)a, (const char*)w, (char*)c, m, n, k);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
