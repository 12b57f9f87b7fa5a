// bi_norm.hip — batch-invariant RMSNorm (gfx950): one wavefront per row, fixed reduction order.
//
// RMSNorm must keep one reduction strategy at every batch size, never a split reduction across
// cores (xitu-tech.com report, section 构建确定性解决方案, RMSNorm item; neican.ai insight page,
// section 技术原理与创新点解析, RMSNorm item: one batch element per core). Here the core is a
// wavefront: row r is read, reduced and written by one wave, which never exchanges data with
// another, so the bits of a row cannot depend on how many rows there are.
//
// HBM-bound: a row is read once (kept in registers up to kCache 16-byte chunks per lane, with
// the matching weight chunks; read again from L2/HBM past that) and written once.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bi_norm.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNormWaves = 4;      // waves (rows in flight) per workgroup
constexpr int kCache = 8;          // 16-byte chunks per lane kept in registers (8 KB rows of bf16)

__device__ __forceinline__ float bf_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ unsigned bf_pack(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 r = {(__bf16)lo, (__bf16)hi};   // round to nearest even
  return __builtin_bit_cast(unsigned, r);
}

// Sum of squares of one 16-byte chunk, elements in ascending order.
template <bool BF> __device__ __forceinline__ float chunk_sq(u32x4 c) {
  float s = 0.f;
  if constexpr (BF) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float a = bf_lo(c[k]), b = bf_hi(c[k]);
      s = __builtin_fmaf(a, a, s);
      s = __builtin_fmaf(b, b, s);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned e = c[k];
      const float a = __builtin_bit_cast(float, e);
      s = __builtin_fmaf(a, a, s);
    }
  }
  return s;
}

// y chunk = (x * r) * w per element, rounded to the element type.
template <bool BF> __device__ __forceinline__ u32x4 chunk_out(u32x4 x, u32x4 w, float r) {
  u32x4 o;
  if constexpr (BF) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = bf_pack((bf_lo(x[k]) * r) * bf_lo(w[k]), (bf_hi(x[k]) * r) * bf_hi(w[k]));
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned xe = x[k], we = w[k];
      o[k] = __builtin_bit_cast(unsigned, (__builtin_bit_cast(float, xe) * r) * __builtin_bit_cast(float, we));
    }
  }
  return o;
}

template <bool BF>
__global__ __launch_bounds__(64 * kNormWaves) void rmsnorm_kernel(const char* x, const char* w, char* y,
                                                                  int rows, int chunks, float hidden,
                                                                  float eps) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * kNormWaves + (threadIdx.x >> 6)));
  const int nw = (int)gridDim.x * kNormWaves;
  for (int r = wv; r < rows; r += nw) {
    const u32x4* xr = (const u32x4*)(x + (size_t)r * chunks * 16);
    u32x4* yr = (u32x4*)(y + (size_t)r * chunks * 16);
    // lane's chunks lane, lane + 64, ...: squares summed in that order
    // (the chunks held in registers are read and written once: non-temporal loads and stores,
    // measurably faster; the weight row is shared by every row and stays cached)
    u32x4 xc[kCache], wc[kCache];
#pragma unroll
    for (int k = 0; k < kCache; ++k) {
      const int ch = lane + 64 * k;
      if (ch < chunks) {
        xc[k] = __builtin_nontemporal_load(xr + ch);
        wc[k] = ((const u32x4*)w)[ch];
      }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kCache; ++k)
      if (lane + 64 * k < chunks) s += chunk_sq<BF>(xc[k]);
    for (int ch = lane + 64 * kCache; ch < chunks; ch += 64) s += chunk_sq<BF>(xr[ch]);
    // fixed butterfly over the 64 lanes: every lane ends with the same total
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    const float rs = 1.0f / __builtin_sqrtf(s / hidden + eps);
#pragma unroll
    for (int k = 0; k < kCache; ++k) {
      const int ch = lane + 64 * k;
      if (ch < chunks) __builtin_nontemporal_store(chunk_out<BF>(xc[k], wc[k], rs), yr + ch);
    }
    for (int ch = lane + 64 * kCache; ch < chunks; ch += 64) yr[ch] = chunk_out<BF>(xr[ch], ((const u32x4*)w)[ch], rs);
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int bi_rmsnorm(const void* x, const void* weight, void* y, int32_t rows, int32_t hidden,
                          int32_t dtype, float eps, hipStream_t stream) {
  if (dtype != 0 && dtype != 1) return 1;
  if (rows < 0 || hidden <= 0 || !(eps >= 0.f) || eps == __builtin_inff()) return 1;
  const int elem = dtype == 1 ? 2 : 4;
  if ((hidden * elem) % 16) return 2;
  if (rows == 0) return 0;
  if (!x || !weight || !y || !aligned16(x) || !aligned16(weight) || !aligned16(y)) return 1;
  const int chunks = hidden * elem / 16;
  // enough waves to keep every CU busy; each wave strides over the rows
  const int64_t need = ((int64_t)rows + kNormWaves - 1) / kNormWaves;
  const int blocks = (int)(need < 4096 ? need : 4096);
  if (dtype == 1)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(blocks), dim3(64 * kNormWaves), 0, stream,
                       (const char*)x, (const char*)weight, (char*)y, rows, chunks, (float)hidden, eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(blocks), dim3(64 * kNormWaves), 0, stream,
                       (const char*)x, (const char*)weight, (char*)y, rows, chunks, (float)hidden, eps);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
