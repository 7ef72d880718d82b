/*
 * miattn — exact tiled attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain device pointers and sizes; no framework types.
 *
 * Operation (prefill): O = softmax(scale * Q K^T + mask) V, computed tile by
 * tile with the online softmax (a running row maximum and denominator; the
 * earlier partial output is rescaled by exp(m_old - m_new) when the maximum
 * grows), so the score matrix is never formed in memory.  Sources, by page:
 *   - "Implementing attention from scratch" (chorfi.xyz), sections Shapes
 *     first (layouts), Why scale by sqrt(D), Masks, Stable softmax, KV caching
 *     (decode, bottom-right causal alignment, grouped-query attention) and
 *     Cost model (decode reads the whole cache);
 *   - "FlashAttention", Transformers in Action section 9.4.1 and Figure 9.8
 *     (exact result, tiles streamed through on-chip memory).
 *
 * Layouts (all row-major, contiguous, head dim fastest; element type given
 * by `dtype`):
 *   q      [B, Hq,  Tq, D]        k, v   [B, Hkv, Tk, D]
 *   o      [B, Hq,  Tq, D]        lse    [B, Hq,  Tq]       (float32)
 *   decode: q [B, Hq, D], k_cache / v_cache [B, Hkv, S_max, D],
 *           o [B, Hq, D], lse [B, Hq]
 * Query head h uses KV head h / (Hq / Hkv) (consecutive query heads share a
 * KV head); Hq must be a multiple of Hkv.
 *
 * Masks.  kv_lens is a DEVICE int32[B] array or NULL.  Sequence b has
 * Lk = clamp(kv_lens[b], 0, Tk) valid keys (NULL: Lk = Tk).  If kv_lens is
 * given and Tq == Tk, the first Lk query rows are valid (self-attention with
 * padding), else all Tq rows are.  Causal: row i sees keys j <= i + Lk - Lq
 * (aligned bottom-right).  A row that is padding or sees no key gets
 * O = 0 and LSE = -inf; no NaN is ever produced.  K/V rows at or past Lk are
 * never read into the result (they may hold anything, NaN included).
 *
 * LSE is the natural-log log-sum-exp of the row's scaled scores over the
 * keys it sees: lse_i = ln sum_j exp(scale * q_i . k_j).
 *
 * Numerics: bf16 inputs are multiplied on the matrix cores with fp32
 * accumulation; softmax statistics and the output accumulator are fp32; the
 * probabilities are rounded to bf16 (round to nearest even) for the P V
 * product and O is rounded to bf16 on store.  fp32 inputs use fp32 matrix
 * instructions end to end.
 *
 * Ownership and concurrency.  The caller owns every buffer (device memory on
 * the current device).  Inputs are read-only; o must not alias q, k or v.
 * The library allocates and frees nothing, never synchronises, and launches
 * on `stream` (a hipStream_t; NULL = the default stream); calls return as
 * soon as the work is queued.  Functions are thread-safe.
 *
 * Alignment.  The kernels move tensors in 16-byte pieces: q, k, v, o, the
 * caches and page pools, dout, dq, dk, dv and every workspace must start on
 * a 16-byte boundary; lse, kv_lens and block_table on a 4-byte boundary
 * (else MIATTN_ERR_ALIGN).  Allocations from hipMalloc (and PyTorch) always
 * are; a view at a storage offset may not be.
 *
 * Errors.  Return 0 on success or a negative MIATTN_ERR_* code.  Arguments
 * are checked before any HIP call; a failed check launches nothing.  Errors
 * never abort the process.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MIATTN_F32 = 0,  /* float32 q/k/v/o */
  MIATTN_BF16 = 1, /* bfloat16 q/k/v/o */
  MIATTN_E4M3 = 2  /* E4M3 codes (the *_fp8 calls); used as a launch-table key only */
};

enum {
  MIATTN_OK = 0,
  MIATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  MIATTN_ERR_SHAPE = -2,       /* size <= 0, Hq % Hkv != 0, non-finite scale(s), or grid too large */
  MIATTN_ERR_UNSUPPORTED = -3, /* D not 64/128, unknown dtype, causal not 0/1 */
  MIATTN_ERR_WORKSPACE = -4,   /* workspace missing or too small */
  MIATTN_ERR_HIP = -5,         /* the HIP runtime refused a launch; see attn_strerror */
  MIATTN_ERR_ALIGN = -6,       /* a pointer is not aligned as required (see Alignment above) */
  MIATTN_ERR_SCRATCH = -7      /* attn_decode_noalloc: the call needs more than its fixed scratch */
};

/*
 * Prefill attention.  q, k, v, o: device pointers of `dtype` elements in the
 * layouts above.  lse: device float32 [B, Hq, Tq] or NULL (not written).
 * scale: any finite value (1/sqrt(D) is the usual one).  causal: 0 or 1.
 * kv_lens: device int32[B] or NULL.  D must be 64 or 128.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
             const int32_t* kv_lens, int dtype, void* stream);

/*
 * Prefill attention on 8-bit floating-point (E4M3) inputs: the FP8 inputs
 * that the self-attention interview question ("Self-Attention:
 * Implementation, Complexity ..."), Follow-up questions, lists among
 * FlashAttention-3's additions.  q, k, v hold one E4M3 code per element
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * 0x7f/0xff NaN, largest magnitude 448) in attn_fwd's layouts, each tensor
 * standing for its codes times its per-tensor scale, so the operation is
 * attn_fwd's with
 *   scores = scale * (q_scale q) . (k_scale k) + mask,   O = P (v_scale V).
 * o is bfloat16 [B, Hq, Tq, D]; lse as attn_fwd (natural log, of those
 * scores).  The scores are exact products of the codes summed in fp32; V is
 * widened to bf16 exactly and P rounded to bf16, as in the bf16 path.  Masks,
 * kv_lens, padding rows and errors as attn_fwd; q_scale, k_scale, v_scale
 * must be finite and scale * q_scale * k_scale finite in float32 (else
 * MIATTN_ERR_SHAPE).  Rows at or past a sequence's length may hold any code.
 */
int attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale,
                 float q_scale, float k_scale, float v_scale, int causal,
                 const int32_t* kv_lens, void* stream);

/* Bytes of device workspace the decode calls need for these sizes (split
 * partials plus a little bookkeeping; not used by the float32 path). */
size_t attn_decode_workspace_size(int B, int Hq, int Hkv, int S_max, int D);

/*
 * One decode step: one new query per (sequence, query head) against a
 * contiguous per-layer KV cache.  kv_lens (device int32[B], required) counts
 * the valid cached keys of each sequence INCLUDING the new token, whose K/V
 * the caller has already written at index kv_lens[b]-1; the query sees keys
 * 0 .. kv_lens[b]-1.  lse: device float32 [B, Hq] or NULL.  workspace:
 * device memory of at least attn_decode_workspace_size(...) bytes, used for
 * split partial results; contents on entry do not matter.  For dtype
 * MIATTN_F32 the workspace is not used and may be NULL.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                int B, int Hq, int Hkv, int S_max, int D, float scale,
                const int32_t* kv_lens, void* workspace, size_t workspace_bytes,
                int dtype, void* stream);

/*
 * attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same operation, arguments (less the
 * workspace), checks and results as attn_decode; the call allocates nothing.
 * The split partials go to a fixed scratch array of
 * attn_decode_noalloc_max_bytes() bytes (96 MiB) that the library holds on
 * each device it runs on until the process ends; a call whose
 * attn_decode_workspace_size(B, Hq, Hkv, S_max, D) exceeds it returns
 * MIATTN_ERR_SCRATCH before any HIP call.  Every call on a device shares that
 * device's array: calls that overlap on one device (e.g. on two streams
 * without ordering between them) race and give wrong results; calls ordered
 * on one stream are fine.  Nothing in the array needs clearing between
 * calls.
 */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        int B, int Hq, int Hkv, int S_max, int D, float scale,
                        const int32_t* kv_lens, int dtype, void* stream);
size_t attn_decode_noalloc_max_bytes(void);

/*
 * One decode step against a paged KV cache: the per-sequence caches live in
 * fixed-size pages of one shared pool, found through a block table (the
 * PagedAttention layout that "Implementing attention from scratch" names in
 * its introduction; the operation is its KV caching section's decode step).
 * Same operation and kv_lens meaning as attn_decode; only where the rows
 * live differs:
 *   k_pages, v_pages  device pools [num_pages, Hkv, page_size, D] (dtype)
 *   block_table       device int32 [B, max_blocks]: logical key j of
 *                     sequence b (j < kv_lens[b]) is row j % page_size of
 *                     page block_table[b * max_blocks + j / page_size].
 * page_size must be a power of two in [8, 65536]; kv_lens[b] is clamped to
 * [0, max_blocks * page_size].  Table entries the call reads (the blocks
 * covering keys < kv_lens[b]) must be valid page numbers; out-of-range
 * entries are clamped into [0, num_pages) on the device (wrong results, no
 * stray access).  Pages not referenced may hold anything, NaN included.
 * workspace: at least attn_decode_workspace_size(B, Hq, Hkv,
 * max_blocks * page_size, D) bytes.  bf16 only.
 */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table, void* o,
                      float* lse, int B, int Hq, int Hkv, int num_pages, int page_size, int max_blocks, int D,
                      float scale, const int32_t* kv_lens, void* workspace, size_t workspace_bytes, int dtype,
                      void* stream);

/*
 * Decode steps on caches of 8-bit floating-point codes (E4M3, the "fn"
 * variant of the OCP 8-bit formats: 1 sign, 4 exponent bits with bias 7,
 * 3 mantissa bits, no infinities, 0x7f/0xff NaN, largest magnitude 448),
 * the FP8 inputs that the self-attention interview question ("Self-Attention:
 * Implementation, Complexity ..."), Follow-up questions, lists among
 * FlashAttention-3's additions.  q, k_cache / k_pages and
 * v_cache / v_pages hold one code byte per element in the same layouts as
 * attn_decode / attn_decode_paged; each tensor stands for its codes times its
 * per-tensor scale (q_scale, k_scale, v_scale: finite, any sign), so the
 * operation is attn_decode's with
 *   scores = scale * (q_scale q) . (k_scale k),   O = P (v_scale V).
 * o is bfloat16 [B, Hq, D]; lse (float32 [B, Hq] or NULL) is the natural-log
 * LSE of those scores.  The scores are exact products of the codes summed in
 * fp32; V is widened to bf16 exactly and P is rounded to bf16 as in the bf16
 * path.  NaN codes past kv_lens[b] are never read into the result.
 * workspace: attn_decode_workspace_size(...) bytes as for the bf16 calls
 * (S_max = max_blocks * page_size for the paged one).  Other arguments,
 * checks and errors as for attn_decode / attn_decode_paged;
 * scale * q_scale * k_scale must be finite in float32 (else
 * MIATTN_ERR_SHAPE).
 */
int attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                    int B, int Hq, int Hkv, int S_max, int D, float scale,
                    float q_scale, float k_scale, float v_scale,
                    const int32_t* kv_lens, void* workspace, size_t workspace_bytes, void* stream);

int attn_decode_paged_fp8(const void* q, const void* k_pages, const void* v_pages, const int32_t* block_table,
                          void* o, float* lse, int B, int Hq, int Hkv, int num_pages, int page_size,
                          int max_blocks, int D, float scale, float q_scale, float k_scale, float v_scale,
                          const int32_t* kv_lens, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_bwd needs: 8 * B * Hq * Tq. */
size_t attn_bwd_workspace_size(int B, int Hq, int Tq);

/*
 * Gradients of the prefill attention (bf16 only; dtype must be MIATTN_BF16,
 * MIATTN_F32 gives MIATTN_ERR_UNSUPPORTED).  Sources: the NumPy
 * tiled-attention build guide, section Extending It (dQ, dK, dV by the chain
 * rule through the softmax), and the self-attention interview question,
 * Task 2 and Hint 2 (the backward recomputes the attention weights tile by
 * tile from Q, K and the saved per-row statistics instead of storing them).
 *
 * Given the forward's inputs q, k, v, its output o and lse (as attn_fwd
 * wrote them, same scale, causal and kv_lens), and dout = dL/dO [B, Hq, Tq,
 * D], writes dq [B, Hq, Tq, D], dk and dv [B, Hkv, Tk, D] (bf16, same
 * layouts as q, k, v):
 *   P = exp(scale * Q K^T + mask - lse),  dV = P^T dO,  dP = dO V^T,
 *   dS = P * (dP - rowsum(dO * O)),  dQ = scale dS K,  dK = scale dS^T Q,
 * with dK and dV of a KV head summed over the query heads sharing it.  Rows
 * with lse = -inf or that are padding get no gradient (dq = 0); keys at or
 * past Lk get dk = dv = 0.  workspace: device memory of at least
 * attn_bwd_workspace_size(B, Hq, Tq) bytes (per-row scratch; contents on
 * entry do not matter); dq, dk, dv must not alias any input.  Every output
 * element is written.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Tq, int Tk, int D, float scale, int causal,
             const int32_t* kv_lens, void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * Launch-choice table.  The NumPy tiled-attention build guide, section
 * Extending It, suggests picking the tile configuration per head size and
 * hardware by measurement, adapting it to varying sequence lengths, and
 * persisting the result; here the compiled kernels take their launch shape
 * as a runtime choice, looked up in this table (the Python binding fills it
 * from the JSON file its tuner writes).  Keys not covered, or no table, use
 * the built-in rule.  Every choice gives a correct result; only speed
 * differs.
 *
 * An entry is MIATTN_TILE_FIELDS int32:
 *   { op, dtype, D, causal, t_lo, t_hi, size_lo, size_hi, v0, v1 }
 *   op    MIATTN_TILE_FWD: attn_fwd (dtype MIATTN_BF16) and attn_fwd_fp8
 *         (MIATTN_E4M3); T = Tk; size = ceil(Tq / 256) * B * Hq; v0 = 0 for
 *         256-row workgroups with one key group, 1 for 128-row workgroups
 *         whose two key groups split the keys; v1 = 1 to pair causal query
 *         tiles long with short, 0 not to, -1 for the built-in rule.
 *   op    MIATTN_TILE_DECODE: the bf16 and E4M3 decode calls, causal = 1;
 *         T = S_max (max_blocks * page_size for the paged calls);
 *         size = B * ceil(S_max / 512) * Hkv * ceil(Hq / Hkv / 16);
 *         v0 = workgroups of the split kernel per compute unit (1..8),
 *         v1 = 0.
 * The first entry whose key matches (t_lo <= T <= t_hi and
 * size_lo <= size <= size_hi) wins.  attn_set_tile_table copies n entries
 * (n <= 256; n = 0 clears the table) and returns MIATTN_ERR_UNSUPPORTED for
 * an invalid entry, leaving the old table in place.  Launches read the table
 * without locking: each call of attn_set_tile_table publishes a new
 * immutable copy, so launches running concurrently see the old or the new
 * table, never a mix; earlier copies stay allocated until the process ends.
 * attn_tile_choice writes the (v0, v1) a launch with that key would use
 * (v1 = -1: the built-in zig-zag rule).
 */
enum { MIATTN_TILE_FWD = 0, MIATTN_TILE_DECODE = 1, MIATTN_TILE_FIELDS = 10 };
int attn_set_tile_table(const int32_t* entries, int n);
int attn_tile_table_size(void);
int attn_tile_choice(int op, int dtype, int D, int causal, long long T, long long size, int32_t* out);

/* Static text for a return code; for MIATTN_ERR_HIP, the last HIP error seen
 * by the calling thread. */
const char* attn_strerror(int code);

/* Library ABI version (incremented on incompatible changes). */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
