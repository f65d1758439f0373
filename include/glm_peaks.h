/* Measured hardware ceilings of the GPU (libglm_peaks.so).
 *
 * Not part of the MoE layer: microbenchmarks whose rates the benchmark
 * reports beside the published MI355X peaks, so that each kernel's roofline
 * fraction can also be read against what the chip sustains at the clock it
 * actually ran, and a shader-clock sampler.  All run on the calling thread's
 * current HIP device, on `stream`; all but the clock sampler block until
 * their timed launches have finished.
 *
 * Return value: a hipError_t value, 0 on success; hipErrorInvalidValue (1)
 * for a null pointer, a non-positive count or a misaligned size.
 */
#ifndef GLM_PEAKS_H
#define GLM_PEAKS_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense MFMA throughput.  `blocks_per_cu` workgroups of four waves per compute
 * unit; every wave issues `iters` x 8 independent register-to-register MFMAs:
 * v_mfma_f32_32x32x16_bf16 when fp8 == 0, the block-scaled
 * v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 operands with unit scales when
 * fp8 == 1.  Outputs (host pointers): *ms the timed launch (HIP events),
 * *flops the floating-point operations it performed (2 per multiply-add),
 * *clock_mhz the shader clock one wave observed over its loop.
 * `scratch`: caller-owned device buffer of at least
 * 16 + 4 * 256 * blocks_per_cu * (number of compute units) bytes. */
int glm_peak_mfma(int fp8, int iters, int blocks_per_cu, void* scratch, float* ms,
                  double* flops, double* clock_mhz, hipStream_t stream);

/* Streaming HBM read bandwidth.  Reads `bytes` (a multiple of 16) from the
 * device buffer `src` (16-byte aligned; make it far larger than the 256 MB
 * last-level cache) with 16-byte non-temporal loads, in two launch shapes
 * (32 workgroups of 256 threads per compute unit with 8 loads in flight per
 * thread; 64 with 4), each once untimed and then `reps` timed times; *ms
 * (host pointer) receives the fastest launch.
 * `scratch`: caller-owned device buffer of at least 2048 * 256 * 4 bytes. */
int glm_peak_hbm_read(const void* src, size_t bytes, int reps, void* scratch, float* ms,
                      hipStream_t stream);

/* The K step of the 256 x 256 bf16 prefill tile with its operands in L2.  One
 * 8-wave workgroup per compute unit runs `iters` (even, > 0) steps of `mode`:
 * 0, the 32 v_mfma_f32_32x32x16_bf16 per wave only; 1, only the step's 64 KB
 * of 16-byte LDS-DMA copies (256 activation and 256 weight rows, 128 bytes
 * each) with the wait and the workgroup barrier of each step; 2, copies,
 * LDS fragment reads and MFMAs, as the grouped GEMM's main loop does them on
 * two 64 KB stages, each wave issuing its 8 copies of the next step at the
 * hand-over; 3, as 2 with each wave's copies spread over the step, two after
 * each of the 4 sub-steps' first row block of MFMAs (the way the prefill
 * kernel issues its weight copies); 4, as 3 without the fragment reads
 * (copies and MFMAs only); 5, fragment reads and MFMAs without copies; 6,
 * MFMAs with the same rows moved through registers (16-byte loads of the next
 * step after the barrier, LDS writes after the step's MFMAs), no fragment
 * reads.  The copies read rows 12 KB apart from `src` (device
 * buffer of at least 512 * 12288 bytes; 2 KB of each row, about 1 MB in all,
 * so they hit L2).  Outputs (host pointers): *us_per_step, the timed launch
 * over `iters` (HIP events); *clock_mhz, the shader clock one wave observed.
 * `scratch`: caller-owned device buffer of at least
 * 16 + 4 * 512 * (number of compute units) bytes. */
int glm_peak_gemm_step(int mode, int iters, const void* src, void* scratch, double* us_per_step,
                       double* clock_mhz, hipStream_t stream);

/* Shader clock while other work runs.  Launches one wave on `stream` (do not
 * wait for it) that, every `period_us` microseconds for `seconds` (0 < seconds
 * <= 10) or until `max_samples` samples, stores the pair (shader clock
 * counter, 100 MHz constant counter) to buf[2i], buf[2i+1], then the number
 * of pairs to buf[2 * max_samples].  Clock in MHz between two samples:
 * 100 * (difference of the first words) / (difference of the second).
 * `buf`: caller-owned device buffer of 2 * max_samples + 1 uint64 words,
 * valid once the stream has passed the probe.  Returns without waiting. */
int glm_peak_clock_probe(double seconds, int period_us, int max_samples, void* buf,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GLM_PEAKS_H */
