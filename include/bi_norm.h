/*
 * bi_norm.h — batch-invariant RMSNorm for MI355X (gfx950), part of libbiattn.so.
 *
 * The write-ups of "Defeating Nondeterminism in LLM Inference" name RMSNorm as one of the three
 * operators that must not change their reduction with the batch: every batch size uses the same
 * data-parallel reduction, never a split reduction across cores (xitu-tech.com report, section
 * 构建确定性解决方案, RMSNorm item); one batch element per core, so each row's reduction stays
 * inside one core (neican.ai insight page, section 技术原理与创新点解析, RMSNorm item).
 *
 * Contract: each row's output is bit-identical whatever the number of rows and the row's
 * position among them, within one build of this library on one device.
 */
#ifndef BI_NORM_H_
#define BI_NORM_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * RMSNorm of rows x [rows][hidden] with weight [hidden] into y [rows][hidden]:
 * y[r][i] = (x[r][i] * (1 / sqrt(sum_i x[r][i]^2 / hidden + eps))) * weight[i], in fp32 with
 * correctly rounded division and square root, y rounded to the element type (nearest even). Each row is reduced by one wavefront: the wavefront's
 * 64 lanes each sum the squares of their 16-byte chunks in ascending chunk order, then a fixed
 * xor butterfly adds the 64 lane sums, so the order never depends on rows.
 * dtype: 0 = fp32, 1 = bf16 (x, weight and y alike). hidden: a positive multiple of 8 (bf16) or
 * 4 (fp32). eps >= 0 and finite. All pointers device memory, 16-byte aligned, caller-owned;
 * x and y may not overlap partially (x == y is allowed: each row is read before it is written).
 * Returns 0 (ok), 1 (invalid argument), 2 (unsupported size) with nothing launched, or 4 when
 * the launch fails. rows == 0 launches nothing.
 */
int bi_rmsnorm(const void* x, const void* weight, void* y, int32_t rows, int32_t hidden,
               int32_t dtype, float eps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BI_NORM_H_ */
