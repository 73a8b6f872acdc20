/*
 * linattn.h -- C ABI of the MI355X (gfx950) kernelized linear-attention library.
 *
 * The operation.  For each (batch b, head h), with phi(x) = elu(x) + 1 (alpha = 1, i.e.
 * x + 1 for x > 0 and exp(x) otherwise) applied elementwise to queries and keys:
 *
 *     out_i = phi(q_i) . KV  /  phi(q_i) . z,   KV = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j)
 *
 * ("Efficient Transformers: Linear Attention and Flash Attention", section "Linear
 * attention: reordering the matmuls, not shrinking them", eq. Attention_i).  The sums run
 * over every key (non-causal) or over keys j <= i (causal: the running state of section
 * "The recurrent view: attention as an RNN", S_t = S_{t-1} + phi(k_t) v_t^T,
 * z_t = z_{t-1} + phi(k_t)).  The feature dimension D equals the head dimension d because
 * phi is elementwise.  There is no 1/sqrt(d) factor and no epsilon in the denominator.
 *
 * Layout.  q, k, v and out are dense row-major [B][H][n][d] (d innermost); for the decode
 * step they are [B][H][d].  The state S is [B][H][d][d] fp32 with S[a][c] = sum phi(k)_a v_c
 * (feature row a, value column c), and z is [B][H][d] fp32.  out has the element type of q.
 *
 * Pointers.  Every tensor pointer is a DEVICE pointer on the HIP device that is current
 * on the calling thread; `stream` is a hipStream_t passed as void* (NULL = the default
 * stream).  Base pointers must be 16-byte aligned.  The caller owns every buffer,
 * including the workspace; the library allocates nothing, frees nothing, keeps no pointer
 * after returning and has no mutable global state.
 *
 * Errors.  Every entry point validates its arguments before launching anything and
 * returns LA_OK or a negative LA_ERR_* code; on an error nothing is written.  Empty
 * shapes (B*H*n == 0) are successful no-ops (except that la_forward_causal_state with n = 0
 * still hands on the state).  Kernels run asynchronously on `stream`:
 * results are valid after the caller synchronises.  A launch failure returns LA_ERR_HIP.
 * Inputs whose phi underflows to zero for every feature (entries below about -87 in fp32)
 * give the IEEE result of 0/0, as the formula would.
 *
 * Supported shapes: d in {64, 128}; element types fp32 and bf16 (state and accumulation are
 * always fp32); causal chunk in {64, 128} for bf16, and for fp32 with d * chunk <= 8192 (d = 64:
 * 64 or 128; d = 128: 64 only -- the fp32 kernel keeps the chunk's phi(K) and V and the
 * transposed state in LDS as two bf16 planes each), else LA_ERR_UNSUPPORTED.
 *
 * Precision.  bf16 inputs: products of bf16 values (the running state and the masked weights
 * rounded to bf16 where they enter a product), fp32 accumulation.  fp32 inputs: every product of
 * two fp32 values is taken on the bf16 matrix cores from two-term splits, x = hi + lo with hi the
 * truncation of x to bf16 and lo the bf16 rounding of the rest (x held to 2^-16 of its size):
 * the four products hi*hi + hi*lo + lo*hi + lo*lo, accumulated in fp32.  A product is within
 * 2^-15 of its size, with errors of either sign, and results stay well inside a relative error of
 * 1e-4.  Infinities and NaN give the result classes of fp32 arithmetic.  The decode step and the
 * normalisers' dot products of the non-causal output compute in fp32 throughout.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 1

/* Element type of q, k, v and out.  The two range markers give the type every int value, so an
 * unknown code passed across the ABI is a defined value, which every entry point rejects with
 * LA_ERR_DTYPE. */
typedef enum {
  LA_DTYPE_F32 = 0,
  LA_DTYPE_BF16 = 1,
  LA_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  LA_DTYPE_RANGE_MAX_ = 2147483647
} la_dtype_t;

enum {
  LA_OK = 0,
  LA_ERR_NULL = -1,        /* a required pointer is NULL while the shape is non-empty   */
  LA_ERR_SHAPE = -2,       /* negative or overflowing dimension                          */
  LA_ERR_DTYPE = -3,       /* unknown element type                                       */
  LA_ERR_UNSUPPORTED = -4, /* d or chunk outside the supported set                      */
  LA_ERR_ALIGN = -5,       /* a base pointer is not 16-byte aligned                      */
  LA_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the *_workspace_bytes size  */
  LA_ERR_ALIAS = -7,       /* out overlaps an input (or the state)                       */
  LA_ERR_HIP = -8,         /* a kernel launch failed                                     */
  LA_ERR_VALUE = -9        /* a scalar argument out of range (FAVOR+ scale)              */
};

/* ABI version of the loaded library (LA_ABI_VERSION at build time). */
int la_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* la_status_string(int status);

/* Bytes of device workspace la_forward_noncausal needs for this shape (0 for an empty
 * shape; (size_t)0 also for unsupported arguments, which the call itself reports). */
size_t la_noncausal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, la_dtype_t dtype);

/*
 * Non-causal forward: every query attends to all n keys of its (b, h).
 *   q, k, v : [B][H][n][d] of `dtype`, read only
 *   out     : [B][H][n][d] of `dtype`, written; must not overlap q, k, v or workspace
 *   workspace, workspace_bytes : device scratch of at least
 *             la_noncausal_workspace_bytes(B, H, n, d, dtype) bytes, any contents (each call
 *             initialises what it uses); it may be reused across calls of any shape, but two
 *             calls that share a workspace must not run concurrently.
 * Two stages ("Efficient Transformers ...", section "Linear attention": the D x d sum and the
 * key sum are built once and shared by every query): split-n partial sums of
 * [phi(K)^T V | phi(K)^T 1] reduced in a fixed order (deterministic), then one pass over
 * the queries.
 */
int la_forward_noncausal(const void* q, const void* k, const void* v, void* out, int64_t B,
                         int64_t H, int64_t n, int64_t d, la_dtype_t dtype, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * la_forward_noncausal for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and the
 * same results (bit for bit), with the slice partials (and their per-head sums) kept in a device
 * array of the library instead of a caller's workspace.  The call allocates nothing and frees nothing.
 *   q, k, v, out, B, H, n, d, dtype, stream : as for la_forward_noncausal
 * The array holds LA_NOALLOC_SCRATCH_BYTES bytes per GPU; it is reserved when the library's code
 * is loaded on a GPU and held until the process ends.  A shape whose partials need more
 * (la_noncausal_workspace_bytes(...) > LA_NOALLOC_SCRATCH_BYTES: B * H above about 4000 at d = 64
 * or 500 at d = 128) returns LA_ERR_WORKSPACE before anything is launched.  Every call on
 * one GPU shares that GPU's array, and each call initialises what it uses: calls that overlap on
 * one GPU (on different streams, or from different threads without ordering) race and may return
 * wrong results.  The first call on a device looks up the array's device address there (a HIP
 * failure is LA_ERR_HIP; a device index of 64 or more is LA_ERR_UNSUPPORTED).
 */
#define LA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int la_forward_noncausal_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B,
                                 int64_t H, int64_t n, int64_t d, la_dtype_t dtype, void* stream);

/* Bytes of device workspace la_forward_causal needs (may be 0). */
size_t la_causal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk,
                                 la_dtype_t dtype);

/*
 * Causal forward: query i attends to keys j <= i (inclusive) of its (b, h).
 *   q, k, v, out : as for la_forward_noncausal
 *   chunk        : 64 or 128 (fp32: d * chunk <= 8192, so 64 at d = 128; others give
 *                  LA_ERR_UNSUPPORTED); the tile of the chunked evaluation.  Within a chunk the masked
 *                  pairwise weights are used directly, earlier tokens enter through the
 *                  running state (S, z) ("The recurrent view"); the result does not depend
 *                  on chunk beyond rounding.
 *   workspace    : at least la_causal_workspace_bytes(...) bytes, same rules as the
 *                  non-causal workspace (may be NULL when that size is 0).
 */
int la_forward_causal(const void* q, const void* k, const void* v, void* out, int64_t B,
                      int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal forward that continues from a given state and hands on the final one (the prefill
 * side of a decode, or one piece of a sequence cut into pieces): with (S0, z0) the state
 * before token 0 ("The recurrent view": S_t = S_{t-1} + phi(k_t) v_t^T from S_{-1} = S0),
 *     out_i = phi(q_i)^T (S0 + sum_{j<=i} phi(k_j) v_j^T) / phi(q_i)^T (z0 + sum_{j<=i} phi(k_j))
 * and (Sn, zn) receive S0 + sum_j phi(k_j) v_j^T and z0 + sum_j phi(k_j) over all n tokens.
 * Running the pieces of a sequence in order, each from the previous piece's final state,
 * gives the outputs and final state of one call over the whole sequence (up to rounding).
 *   S0, z0 : [B][H][d][d] and [B][H][d] fp32, read only; both NULL for the zero state
 *   Sn, zn : [B][H][d][d] and [B][H][d] fp32, written; both NULL to skip.  They must not
 *            overlap any other argument (no update in place of S0, z0): the final state is
 *            written while other workgroups may still read the initial one.
 *   other arguments and the workspace: as for la_forward_causal, which is this call with
 *   all four state pointers NULL.  With n = 0 the call writes Sn, zn = S0, z0 (zeros when
 *   S0 is NULL) and reads no other tensor.  Giving only one pointer of a pair is LA_ERR_NULL.
 */
int la_forward_causal_state(const void* q, const void* k, const void* v, void* out,
                            const float* S0, const float* z0, float* Sn, float* zn, int64_t B,
                            int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two stages of la_forward_causal, callable on their own (a caller can time them apart,
 * or supply segment states computed elsewhere, e.g. on another device that holds the earlier
 * part of the sequence).  Each head's sequence is cut into segments of `seg_len` tokens
 * (a positive multiple of chunk); segment s covers tokens [s*seg_len, min(n, (s+1)*seg_len)).
 *
 * la_causal_plan: the seg_len la_forward_causal uses for this shape (1 segment when the
 * batch alone fills the GPU).  Returns LA_OK and writes *seg_len, or an error code.
 *
 * la_state_sums: for s < nseg writes sums[b][h][s] = [S | z] (fp32, d*d values of
 * S = sum phi(k_j) v_j^T row-major, then d values of z = sum phi(k_j)) over the tokens of
 * segment s ("The recurrent view": the state is a plain sum over tokens, so it splits over
 * segments).  sums is [B][H][nseg][d*d + d] fp32 and must not overlap k, v or workspace.
 * Needs la_state_sums_workspace_bytes(...) bytes of workspace (same rules as above; when
 * that size is 0 the workspace may be NULL).  Requires 1 <= nseg and (nseg-1)*seg_len < n.
 *
 * la_causal_segments: the chunked causal pass.  Segment s starts from the state
 * sum_{s' < s} sums[b][h][s'] (zero for s = 0), so sums must hold ceil(n/seg_len) - 1 entries
 * per head: [B][H][ceil(n/seg_len) - 1][d*d + d] (may be NULL when that count is 0).
 */
int la_causal_plan(int64_t B, int64_t H, int64_t n, int64_t d, int64_t chunk, la_dtype_t dtype,
                   int64_t* seg_len);

size_t la_state_sums_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, la_dtype_t dtype,
                                     int64_t seg_len, int64_t nseg);

int la_state_sums(const void* k, const void* v, float* sums, int64_t B, int64_t H, int64_t n,
                  int64_t d, la_dtype_t dtype, int64_t seg_len, int64_t nseg, void* workspace,
                  size_t workspace_bytes, void* stream);

int la_causal_segments(const void* q, const void* k, const void* v, void* out,
                       const float* sums, int64_t B, int64_t H, int64_t n, int64_t d,
                       int64_t chunk, la_dtype_t dtype, int64_t seg_len, void* stream);

/*
 * Variable-length batches: nseq sequences of n_s tokens each, every one laid out as the fixed
 * layout's [H][n_s][d] block, the blocks packed back to back (sequence s starts at element
 * H * cu_seqlens[s] * d).  cu_seqlens is a HOST array of nseq + 1 offsets in tokens:
 * cu_seqlens[0] = 0, nondecreasing, n_s = cu_seqlens[s + 1] - cu_seqlens[s] (0 allowed);
 * nseq <= 256 (LA_ERR_UNSUPPORTED above).  The library reads it during the call only.  Each
 * sequence's result is that of the fixed-length call on it alone (up to rounding: the work is
 * cut into slices and segments planned for the longest sequence).  q, k, v and out are
 * [sum_s H n_s d] elements; other arguments and the workspace rules as for the fixed-length
 * calls, with the workspace sizes below.  Bad offsets (not starting at 0, decreasing) give
 * LA_ERR_SHAPE, a NULL cu_seqlens LA_ERR_NULL.
 */
size_t la_noncausal_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t nseq, int64_t H,
                                           int64_t d, la_dtype_t dtype);

int la_forward_noncausal_varlen(const void* q, const void* k, const void* v, void* out,
                                const int64_t* cu_seqlens, int64_t nseq, int64_t H, int64_t d,
                                la_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);

size_t la_causal_varlen_workspace_bytes(const int64_t* cu_seqlens, int64_t nseq, int64_t H,
                                        int64_t d, int64_t chunk, la_dtype_t dtype);

int la_forward_causal_varlen(const void* q, const void* k, const void* v, void* out,
                             const int64_t* cu_seqlens, int64_t nseq, int64_t H, int64_t d,
                             int64_t chunk, la_dtype_t dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * One recurrent decode step for B*H independent heads, in place on the state
 * ("The recurrent view"; the fixed-size state of Active recall A5):
 *     S += phi(k) v^T ;  z += phi(k) ;  out = phi(q)^T S / phi(q)^T z
 * (the new token is folded in first, then read with q).
 *   q, k, v : [B][H][d] of `dtype`, read only
 *   S       : [B][H][d][d] fp32, read and written in place
 *   z       : [B][H][d] fp32, read and written in place
 *   out     : [B][H][d] of `dtype`, written; must not overlap q, k, v, S or z
 * The state is the whole checkpoint: copying S and z out and back resumes bit-exactly.
 */
int la_decode_step(const void* q, const void* k, const void* v, float* S, float* z, void* out,
                   int64_t B, int64_t H, int64_t d, la_dtype_t dtype, void* stream);

/*
 * la_decode_step for the sequences whose flag is set: active is a DEVICE array of B bytes
 * (nonzero = active), read by the kernel, so it may change from step to step without a host
 * synchronisation.  For an inactive sequence the state (S, z) and out are left as they were.
 * active must not be NULL (LA_ERR_NULL) nor overlap out, S or z.
 */
int la_decode_step_masked(const void* q, const void* k, const void* v, float* S, float* z,
                          void* out, const uint8_t* active, int64_t B, int64_t H, int64_t d,
                          la_dtype_t dtype, void* stream);

/* ---------------------------------------------------------------------------------------
 * FAVOR+ feature map.  "Efficient Transformers: Linear Attention and Flash Attention" (section
 * "Linear attention: reordering the matmuls, not shrinking them") names FAVOR+ (Choromanski et
 * al., "Rethinking Attention with Performers") as the non-negative random-feature alternative to
 * elu + 1 whose inner products approximate the softmax kernel exp(x . y).  Its positive random
 * features are used here:
 *     phi(x) = exp(W x' - |x'|^2 / 2) / sqrt(m),   x' = scale * x,
 * with W the [m][d] projection (rows are Gaussian directions; the caller draws it, i.i.d. or in
 * orthogonal blocks, and may redraw it between calls).  phi(q) . phi(k) then estimates
 * exp(scale^2 q . k); scale = d^(-1/4) gives the kernel of softmax attention.  The attention is
 * eq. Attention_i with this phi (out_i = phi(q_i)^T S / phi(q_i)^T z, S = sum_j phi(k_j) v_j^T
 * [m][d], z = sum_j phi(k_j) [m]), over all keys or over j <= i.
 *
 * Supported: bf16 only (q, k, v, W, out; fp32 is LA_ERR_UNSUPPORTED), d = 64 with m in
 * {64, 128, 256}, d = 128 with m in {64, 128} (m * d <= 16384); other (d, m) pairs return
 * LA_ERR_UNSUPPORTED.  scale must be positive and finite (LA_ERR_VALUE).  W is read only, 16-byte
 * aligned, and shared by all heads.
 *
 * State with a log-scale.  The exponents of phi leave fp32's range for large inputs, so a state
 * handed across the ABI is (S [m][d], z [m], c) with the true state exp(c) * (S, z).  The empty
 * state is S = 0, z = 0, c = -infinity.  The kernels keep every stored value within range by
 * moving the scale into c (exact rewriting, nothing is dropped).
 * ------------------------------------------------------------------------------------- */

/* Workspace bytes of la_favor_forward_noncausal for this shape (0 for an empty or invalid one). */
size_t la_favor_noncausal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                                          la_dtype_t dtype);

/*
 * Non-causal FAVOR+ attention: out_i = phi(q_i)^T S / phi(q_i)^T z over all n keys of the head.
 *   q, k, v, out : [B][H][n][d] bf16; out must not overlap q, k, v, w or the workspace
 *   w            : [m][d] bf16 projection
 *   workspace    : at least la_favor_noncausal_workspace_bytes bytes, 16-byte aligned, owned by
 *                  the caller; its contents on entry do not matter
 */
int la_favor_forward_noncausal(const void* q, const void* k, const void* v, const void* w,
                               void* out, int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                               float scale, la_dtype_t dtype, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Workspace bytes of la_favor_forward_causal (0: none needed, or an invalid shape). */
size_t la_favor_causal_workspace_bytes(int64_t B, int64_t H, int64_t n, int64_t d, int64_t m,
                                       int64_t chunk, la_dtype_t dtype);

/*
 * Causal FAVOR+ attention (j <= i), chunked ("The recurrent view": the prefix sums S_i, z_i split
 * at each chunk start into the carried state and the masked pairwise part inside the chunk).
 *   q, k, v, out : [B][H][n][d] bf16; w : [m][d] bf16
 *   chunk        : 64, or 128 when m <= 128 (others LA_ERR_UNSUPPORTED); the result does not
 *                  depend on it beyond rounding
 *   Sn, zn, cn   : all NULL, or all given: receive the state after token n-1 as
 *                  exp(cn) * (Sn [B][H][m][d], zn [B][H][m]) fp32 (Sn 16-byte aligned, zn and cn
 *                  4-byte aligned), the input of la_favor_decode_step; for n = 0 the empty state
 *                  is written and q, k, v, w, out are not read.  Giving only some is LA_ERR_NULL.
 *   workspace    : la_favor_causal_workspace_bytes bytes (may be NULL when that is 0)
 * No output (out, Sn, zn, cn) may overlap another output, an input or the workspace.
 */
int la_favor_forward_causal(const void* q, const void* k, const void* v, const void* w, void* out,
                            float* Sn, float* zn, float* cn, int64_t B, int64_t H, int64_t n,
                            int64_t d, int64_t m, int64_t chunk, float scale, la_dtype_t dtype,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * One FAVOR+ decode step for B*H heads, in place on the state ("The recurrent view"):
 *     S += phi(k) v^T ;  z += phi(k) ;  out = phi(q)^T S / phi(q)^T z   (update first)
 * with the state kept as exp(c) * (S, z) (c moves to the larger exponent when a key needs it).
 *   q, k, v, out : [B][H][d] bf16
 *   w            : [m][d] bf16
 *   S [B][H][m][d], z [B][H][m], c [B][H] : fp32, read and written in place; S 16-byte aligned,
 *                  z and c 4-byte aligned; start from the empty state (zeros, c = -infinity) or
 *                  from a state written by la_favor_forward_causal
 * No two of out, S, z, c may overlap, nor any of them q, k, v or w (LA_ERR_ALIAS).
 */
int la_favor_decode_step(const void* q, const void* k, const void* v, const void* w, float* S,
                         float* z, float* c, void* out, int64_t B, int64_t H, int64_t d, int64_t m,
                         float scale, la_dtype_t dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
