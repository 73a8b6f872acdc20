/*
 * la_ceiling.h -- memory-system measurements that bound the linear-attention kernels.
 *
 * A memory-bound kernel's time is at least its bytes over the bandwidth the memory system
 * delivers to that access pattern (Hoefler, "Let's Stop Calling Everything 'Linear Attention'",
 * section 2, memory-load traffic: t_mem >= T_mem / B_effective).  B_effective is itself a
 * measurement: these calls move known bytes with the simplest kernels that have a given
 * pattern, and compute a result that can be checked, so that nothing is optimised away.  They
 * are measurement tools, not part of the attention computation.
 *
 * Pointers are device pointers on the current HIP device, 16-byte aligned; `stream` is a
 * hipStream_t passed as void* (NULL = default stream).  Status codes are those of linattn.h
 * (LA_OK, LA_ERR_NULL, LA_ERR_SHAPE, LA_ERR_ALIGN, LA_ERR_ALIAS, LA_ERR_UNSUPPORTED, LA_ERR_HIP).
 * The library allocates nothing.
 */
#ifndef LA_CEILING_H
#define LA_CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Plain device copy of `bytes` (a positive multiple of 16): dst = src.  One 16-byte piece per
 * thread, non-temporal both ways, one 256-thread workgroup per 4 KB of the buffer (the fastest
 * copy pattern measured on the device).  src and dst must not overlap; a buffer of more than
 * INT_MAX * 4 KB is LA_ERR_SHAPE.
 */
int la_ceiling_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Read-only stream over `bytes` (a positive multiple of 16): every 16-byte piece of src is read
 * once, non-temporally, each of la_ceiling_read_sink_words() workgroups streaming one contiguous
 * range; sink[w] (uint32) receives the XOR of the 32-bit words workgroup w read, so the result is
 * checkable.  sink must not overlap src.
 */
size_t la_ceiling_read_sink_words(void);
int la_ceiling_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * The chunked causal kernel's memory pattern with arithmetic that is just a sum: for bf16
 * [B][H][n][d] tensors (d = 128), out = q + k + v elementwise (fp32 sum of the three bf16
 * values, rounded to nearest even).  Workgroups, chunks and accesses follow causal_bf16 at
 * d = 128, chunk 128: one 512-thread workgroup per (head, segment of seg_len tokens), one per
 * compute unit (its LDS use is the same size class); each walks its segment in 128-token chunks
 * with the next chunk's k, v and q rows in flight (non-temporal loads; k and v as whole 256-byte
 * rows, q in 16-row x 64-byte pieces), stages k and v through LDS and stores out in 16-row x
 * 64-byte pieces.  seg_len: a positive multiple of 128 (la_causal_plan gives the causal kernel's).
 * out must not overlap q, k or v.
 */
int la_ceiling_causal_pattern(const void* q, const void* k, const void* v, void* out, int64_t B,
                              int64_t H, int64_t n, int64_t d, int64_t seg_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_CEILING_H */
