/*
 * attn_probes.h — C ABI of libattn_probes.so, the device-ceiling probes that the benchmark
 * reports beside the attention kernels' roofline fractions (measurement only; no attention
 * arithmetic lives here and the attention library does not use it).
 *
 * The roofline denominators of the attention kernels are the vendor's spec figures (8 TB/s of
 * HBM3E, 2.5 PFLOP/s of dense bf16 MFMA at 2.4 GHz). These probes measure what the device
 * delivers for the two operations the kernels are bound by, with the instruction forms the
 * kernels use: 16-byte global loads streaming from HBM (what the split-KV decode kernel does
 * with the paged K/V rows) and back-to-back v_mfma_f32_32x32x16_bf16 (the prefill kernel's QK^T
 * and PV products), plus the shader clock under that MFMA load, and the LDS read rate of the
 * prefill kernel's two LDS read forms (its K and V^T operand reads).
 *
 * Conventions: device pointers are caller-owned; kernels are queued on `stream` (a hipStream_t,
 * NULL = the null stream) and the call returns once they are queued. Return value: 0 on success,
 * 1 for an argument error (checked on the host before anything is queued), 2 when the launch
 * fails.
 */
#ifndef ATTN_PROBES_H_
#define ATTN_PROBES_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_probe_read_stream: read `bytes` bytes of device memory at `src` (16-byte aligned, bytes a
 * positive multiple of 16 KiB) once, with 16-byte loads, `workgroups` workgroups of 256 threads
 * walking the buffer grid-stride with 4 loads in flight per thread; nontemporal != 0 marks
 * every load non-temporal (the streaming hint the decode kernel's K/V loads carry). The loaded
 * words are folded (xor) into one uint32 per thread written to sink[workgroups * 256], so no
 * load can be dropped. Bytes moved: `bytes` read, workgroups * 1 KiB written.
 */
int32_t attn_probe_read_stream(const void* src, uint64_t bytes, uint32_t* sink,
                               int32_t workgroups, int32_t nontemporal, void* stream);

/*
 * attn_probe_mfma_loop: `workgroups` workgroups of 8 waves (two per SIMD, as the prefill
 * kernel runs) each issue `iters` rounds of 4 independent v_mfma_f32_32x32x16_bf16 products per
 * wave (32 * 32 * 16 * 2 = 32768 flops each), so the work is
 * workgroups * 8 * iters * 4 * 32768 flops. Each wave writes the sum of its accumulators to
 * sink[workgroups * 8]. Wave 0 of each workgroup records, at its start and end, the shader
 * clock counter (s_memtime) and the constant 100 MHz reference counter (s_memrealtime):
 * clocks[4 * w + 0..3] = start shader, end shader, start reference, end reference, so the mean
 * shader clock under this load is 100 MHz * d(shader) / d(reference).
 */
int32_t attn_probe_mfma_loop(uint64_t* clocks, float* sink, int32_t workgroups, int32_t iters,
                             void* stream);

/*
 * attn_probe_lds_read: `workgroups` workgroups of 8 waves, each with a 64 KiB LDS tile filled
 * once; every wave then issues `iters` rounds of 8 independent LDS reads and folds what it reads
 * into one uint32 per thread, written to sink[workgroups * 512]. transposing == 0:
 * ds_read_b128 (16 bytes per lane, 1 KiB per read); transposing != 0: ds_read_b64_tr_b16
 * (8 bytes per lane, 512 bytes per read) with the prefill kernel's V^T addressing for
 * head_size 128. Bytes read per workgroup: 8 * iters * 8 * (1024 or 512). clocks as for
 * attn_probe_mfma_loop (wave 0: start and end shader clock, start and end 100 MHz reference).
 */
int32_t attn_probe_lds_read(uint64_t* clocks, uint32_t* sink, int32_t workgroups, int32_t iters,
                            int32_t transposing, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBES_H_ */
