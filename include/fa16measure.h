/*
 * fa16measure — measurement aids for the fa16attn benchmark on MI355X
 * (gfx950). Nothing here is part of the attention method: this small library
 * (libfa16measure.so) exists so that a benchmark can report, beside the
 * published peak, the matrix throughput the chip actually sustains.
 * The attention library (fa16attn.h) neither declares nor links it.
 *
 * Conventions as fa16attn.h: device pointers, caller-owned memory, the call
 * enqueues on `stream` (a hipStream_t; NULL = the null stream), validates its
 * arguments on the host before any HIP call and never synchronises.
 */
#ifndef FA16MEASURE_H
#define FA16MEASURE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes: 0 success, 1 a NULL pointer, 2 a size out of range,
 * FAM_ERR_HIP + e for HIP error e from the launch. */
enum fam_status { FAM_OK = 0, FAM_ERR_NULL = 1, FAM_ERR_SHAPE = 2, FAM_ERR_HIP = 1000 };

/*
 * One launch of a kernel that issues only FP16 MFMAs
 * (v_mfma_f32_32x32x16_f16) on operands that vary from lane to lane:
 * 512 workgroups of 256 threads (two per CU), each wave running iters x 4
 * MFMAs, i.e. 512 * 4 * iters * 4 * 32768 FLOP. Its rate is the FP16 matrix
 * throughput the chip sustains on varied data.
 * out: device FP32 [512 * 256] (one value per thread, caller-owned).
 * Domain: 1 <= iters <= 2^20.
 */
int fa_mfma_ceiling(int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA16MEASURE_H */
