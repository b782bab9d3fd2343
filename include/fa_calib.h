/*
 * fa_calib.h -- calibration kernels for AMD Instinct MI355X (gfx950): the empirical
 * ceilings the attention kernels of fa.h are measured against, next to the published
 * peaks (dense bf16 matrix throughput, HBM bandwidth), and the shader clock.
 *
 * These are measurement tools, not part of the attention path.  Same conventions as fa.h:
 * C linkage, DEVICE pointers owned by the caller, nothing allocated, freed or synchronised
 * inside; each call validates, enqueues on `stream` (a hipStream_t or NULL) and returns
 * 0 on success, 1 for a NULL pointer, 2 for a bad size, 6 when the launch fails.
 */
#ifndef FA_MI355X_CALIB_H
#define FA_MI355X_CALIB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fa_calib_mfma -- the matrix-core ceiling: `blocks` workgroups of 8 waves (two per SIMD,
 * as the prefill kernels run), each wave issuing `iters` rounds of four independent
 * 32x32x16 bf16 MFMAs (fp32 accumulate) on register operands, nothing else.
 * Work = blocks * 8 * iters * 4 * 32768 FLOP.
 *   sink:   >= blocks * 512 floats (written, so the products are not optimised away)
 *   cycles: >= 2 * blocks uint64 (per workgroup: shader-clock ticks (s_memtime), then 100 MHz
 *           real-time ticks (s_memrealtime), from the start of its loop to the end of its last wave)
 *   blocks >= 1, iters >= 1.
 */
int fa_calib_mfma(float* sink, uint64_t* cycles, int blocks, int iters, void* stream);

/*
 * fa_calib_mfma_valu -- how far vector work hides under matrix work when the same waves
 * issue both, as in the attention loops: the workgroups of fa_calib_mfma, each wave running
 * `iters` rounds of (mfma ? four 32x32x16 bf16 MFMAs : nothing) followed by `fmas` fp32
 * FMAs in eight independent chains.  mfma in {0, 1}, fmas in {0, 24, 48}, not both 0
 * (mfma = 1, fmas = 0 is the loop of fa_calib_mfma).  Time the three variants of one
 * `fmas` count: if the vector work hid completely, mixed = MFMA-only; if not at all,
 * mixed = MFMA-only + FMA-only.  Same buffers and return codes as fa_calib_mfma.
 */
int fa_calib_mfma_valu(float* sink, uint64_t* cycles, int blocks, int iters, int mfma, int fmas, void* stream);

/*
 * fa_calib_stream_read -- the HBM read ceiling for a one-pass stream, in the access
 * pattern of the decode kernel: `blocks` workgroups of 256 threads read `bytes` bytes of
 * `buf` once, 16 bytes per lane per load, two loads in flight per lane, nontemporal
 * (the lines are not kept in the caches).
 *   buf: device buffer, 16-byte aligned; bytes a multiple of 16 (>= 16).
 *   sink: >= blocks * 256 floats.  blocks >= 1.
 */
int fa_calib_stream_read(const void* buf, size_t bytes, float* sink, int blocks, void* stream);

/*
 * fa_calib_clock -- the shader clock: one wave reads the shader-clock counter (s_memtime)
 * and the 100 MHz real-time counter (s_memrealtime), spins until `spin_ticks` real-time
 * ticks have passed (at most 2^24 loop iterations), and reads both again.
 *   out: >= 2 uint64: out[0] = shader-clock cycles, out[1] = real-time ticks elapsed;
 *   clock in MHz = 100 * out[0] / out[1].  1 <= spin_ticks <= 10^7 (0.1 s).
 */
int fa_calib_clock(uint64_t* out, int spin_ticks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_CALIB_H */
