/*
 * bi_gemm.h — batch-invariant GEMM for MI355X (gfx950), part of libbiattn.so.
 *
 * The write-ups of "Defeating Nondeterminism in LLM Inference" make matrix multiplication batch
 * invariant by dropping the Split-K strategies that adapt to the input size and using one fixed
 * tile configuration for every shape (xitu-tech.com report, section 构建确定性解决方案, matrix
 * multiplication item; neican.ai insight page, section 技术原理与创新点解析, matmul item), at a
 * cost of about 20% against the vendor library (neican.ai insight page, same section).
 *
 * Contract: each output element is bit-identical whatever M (the number of token rows) and the
 * row's position among them, within one build of this library on one device.
 */
#ifndef BI_GEMM_H_
#define BI_GEMM_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * C[M][N] = A[M][K] W[N][K]^T (a linear layer: activations times the transpose of an
 * [out][in] weight), bf16 inputs, fp32 accumulation. One workgroup owns a tile of C (M <= 16
 * and K >= 8192: 32 rows x 32 columns, one wave, operands straight from memory; else 256 x 256
 * when there are at least 160 such tiles and N is a multiple of 256; else 128 x 128, or 64 x 64
 * when there would be fewer than 256 tiles of 128 x 128) and walks the
 * whole of K as MFMA 32x32x16 k-substeps in ascending order into one fp32 accumulator per
 * element: no split of K, and the same per-element order for every M and every tile shape,
 * so C[i][j] depends on row i of A and row j of W only.
 * c_dtype: 0 = fp32, 1 = bf16 (round to nearest even). Sizes: M >= 0 any; N a positive multiple
 * of 128; K a positive multiple of 64 below 2^22. A, W, C: device memory, row-major, 16-byte aligned,
 * caller-owned; C must not overlap A or W. Returns 0 (ok), 1 (invalid argument), 2 (unsupported
 * size) with nothing launched, or 4 when the launch fails. M == 0 launches nothing.
 */
int bi_gemm(const void* a, const void* w, void* c, int32_t m, int32_t n, int32_t k,
            int32_t c_dtype, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_GEMM_H_ */
