/*
 * fa.h -- C ABI of a fused, tiled, exact scaled-dot-product attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h, for every query row i):
 *
 *   scores_ij = scale * sum_d q[b,h,i,d] * k[b,h,j,d]
 *   causal:     scores_ij = -inf for j > i            (key j kept iff j <= i)
 *   o[b,h,i,:] = sum_j softmax_j(scores_i.) * v[b,h,j,:]
 *   lse[b,h,i] = log sum_j exp(scores_ij)              (natural log)
 *
 * This is the five-step naive attention (matmul, scale, masked_fill with -inf,
 * softmax, matmul) of "Profiling in PyTorch (Part 3): Attention is all you
 * profile", section "Naive attention", with the causal keep-matrix built as a
 * lower triangle as in that page's "Math backend" section.  It is evaluated
 * the way that page's "Why flash attention exists" section and the
 * "FlashAttention-2" blog ("FlashAttention-2 Optimizations": causal masking,
 * parallelism over sequence length, work split between waves by query rows)
 * describe: key/value tiles are streamed through on-chip memory with a running
 * softmax, and the seq x seq score matrix never reaches device memory.  The
 * per-row log-sum-exp output is not described on the pages; it is the natural
 * log of the softmax denominator, scale included.
 *
 * Layout: q, k, v and o are dense row-major [B, H, S, D] tensors with D
 * innermost, i.e. element (b,h,s,d) is at ((b*H + h)*S + s)*D + d -- the
 * [batch, heads, seq, head_dim] layout of the naive-attention listing on the
 * same page, consumed as-is (no transposes).  lse is dense float32 [B, H, S].
 * Self-attention only: queries and keys share the one length S.
 *
 * Ownership and memory: every pointer is device memory owned by the caller.
 * The library never allocates, frees or keeps a pointer beyond the call.
 * q, k, v are only read; o and lse are fully overwritten and never read.
 * o and lse must not overlap q, k, v or each other.  q, k, v, o must be 16-byte
 * aligned; lse 4-byte aligned.
 *
 * Asynchrony: the work is enqueued on `stream` (a hipStream_t; NULL means the
 * default stream) and the call returns without synchronising.  The library
 * keeps no state, so concurrent calls on different streams are safe.
 *
 * Errors: arguments are validated on the host before any HIP call.  On a
 * validation error nothing is enqueued and the outputs are untouched.  The
 * functions never throw and never print.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point (plain int in the ABI). */
enum fa_status {
    FA_OK          = 0, /* enqueued */
    FA_ERR_NULL    = 1, /* a tensor pointer is NULL */
    FA_ERR_SHAPE   = 2, /* B, H, S (Sq, Sk, G) < 1, or a size/offset overflows */
    FA_ERR_HEADDIM = 3, /* D not one of 64, 128, 256 */
    FA_ERR_SCALE   = 4, /* scale not finite (NaN or +-inf) */
    FA_ERR_CAUSAL  = 5, /* causal not 0 or 1 */
    FA_ERR_ALIGN   = 6, /* q/k/v/o not 16-byte aligned or lse not 4-byte aligned */
    FA_ERR_ALIAS   = 7, /* o or lse overlaps an input or each other */
    FA_ERR_LAUNCH  = 8, /* the HIP launch (or a HIP query before it) failed */
    FA_ERR_SCRATCH = 9  /* fa_bwd_noalloc: B*H*S above FA_BWD_SCRATCH_ROWS */
};

/* Rows (B*H*S) the library's fixed backward scratch array holds: one float32
 * per row, 8 MiB on each GPU the library runs fa_bwd_noalloc on. */
#define FA_BWD_SCRATCH_ROWS (1 << 21)

/*
 * fa_fwd -- bf16 attention forward.
 *   q, k, v : bf16 [B,H,S,D] inputs (device).
 *   o       : bf16 [B,H,S,D] output (device), rounded to nearest even from the
 *             float32 accumulator.
 *   lse     : float32 [B,H,S] output (device), natural-log log-sum-exp.
 *   B, H, S : batch, heads, sequence length (>= 1).
 *   D       : head dimension, one of 64, 128, 256.
 *   causal  : 1 = key j visible to query i iff j <= i; 0 = all keys.
 *   scale   : score multiplier, any finite value (usually 1/sqrt(D)).  A
 *             negative scale is computed exactly as |scale| on negated q; a
 *             zero scale gives every visible key the same weight (O = mean of
 *             the visible v rows, lse = log of their count).
 *   stream  : hipStream_t to enqueue on (NULL = default stream).
 * Arithmetic: bf16 products with float32 accumulation for both contractions;
 * the softmax (running max, exponentials, running sum) is float32; the softmax
 * weights are rounded to bf16 before they multiply v.
 * Returns an fa_status value.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int S, int D, int causal, float scale, void* stream);

/*
 * fa_fwd_f32 -- the same operation on float32 q, k, v, o.  All arithmetic is
 * float32 (float32 matrix-core products and accumulation, float32 softmax
 * weights).  Arguments, layout, ownership and errors as for fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int S, int D, int causal, float scale, void* stream);

/*
 * fa_fwd_kv -- bf16 attention of Sq queries against Sk keys (chunked prefill
 * against a cached prefix, decode), with the causal mask aligned
 * bottom-right.
 *   q, o    : bf16 [B,H,Sq,D]; k, v : bf16 [B,H,Sk,D]; lse : float32 [B,H,Sq].
 *   Sq, Sk  : query rows and keys per (batch, head), >= 1.
 * The queries are taken to be the last Sq positions of the Sk-position
 * sequence: with causal = 1, key j is visible to query i iff
 * j <= i + (Sk - Sq).  This is the lower-triangular keep-matrix of
 * "Profiling in PyTorch (Part 3): Attention is all you profile", section
 * "Math backend", with its diagonal moved by Sk - Sq (the pages treat only
 * Sq = Sk).  A row with no visible key (i < Sq - Sk) gets the result that
 * section's safe softmax gives: o row = 0, lse = -inf.  With causal = 0
 * every query sees all Sk keys.  fa_fwd(..., S, ...) is fa_fwd_kv with
 * Sq = Sk = S.  Arithmetic, ownership, alignment and errors as for fa_fwd
 * (FA_ERR_SHAPE also when Sq or Sk < 1).  The work is split over query
 * tiles only, so a call with few query rows (decode) uses few workgroups.
 */
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Sq, int Sk, int D, int causal, float scale, void* stream);

/*
 * fa_merge -- combine G results computed over disjoint key sets of the same
 * queries (split over keys: shards of a long key sequence, or a cached prefix
 * and a new chunk) into the result over their union.
 *   o_parts   : bf16 [G,B,H,S,D]   part g's output (device), e.g. from fa_fwd_kv.
 *   lse_parts : float32 [G,B,H,S]  part g's natural-log LSE; -inf where a
 *               row saw no key in that part.
 *   o, lse    : bf16 [B,H,S,D] and float32 [B,H,S] results (device).
 *   G >= 1 parts; D one of 64, 128, 256.
 * Per row: lse = log sum_g exp(lse_g), o = sum_g exp(lse_g - lse) o_g,
 * float32 weights and sums, o rounded to nearest even.  Parts whose weight is
 * 0 (lse_g = -inf, or underflow) are skipped and their o is not read; a row
 * with lse_g = -inf in every part gives o = 0, lse = -inf.  This identity
 * follows from the definition of softmax over a union of key sets; it is the
 * reason the per-row LSE is an output.  o_parts, o 16-byte aligned; lse_parts,
 * lse 4-byte aligned; the outputs must not overlap the inputs or each other.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE (G, B, H or S < 1, or a size overflows),
 * FA_ERR_HEADDIM, FA_ERR_ALIGN, FA_ERR_ALIAS, FA_ERR_LAUNCH.
 */
int fa_merge(const void* o_parts, const float* lse_parts, int G, int B, int H, int S, int D,
             void* o, float* lse, void* stream);

/*
 * fa_bwd -- bf16 attention backward: gradients of the fa_fwd output with
 * respect to q, k and v, for an incoming gradient dout of o.
 *   q, k, v : bf16 [B,H,S,D] inputs of the forward call (device).
 *   o, lse  : that call's outputs (bf16 [B,H,S,D], float32 [B,H,S]).
 *   dout    : bf16 [B,H,S,D] gradient of the loss with respect to o.
 *   dq, dk, dv : bf16 [B,H,S,D] results (device), fully overwritten.
 *   delta   : float32 [B,H,S] buffer owned by the caller, overwritten with
 *             rowsum(dout * o) (an intermediate the kernels share; it is an
 *             output so that the call itself allocates nothing).
 *   D       : 64, 128 or 256.
 *   B, H, S, causal, scale, stream : as for fa_fwd (same values as the
 *             forward call).
 * Computes, with P = exp(scale * q k^T - lse) (masked entries 0):
 *   dv = P^T dout;  dS = P * (dout v^T - delta);  dq = scale * dS k;
 *   dk = scale * dS^T q
 * -- the gradient of the operation described for fa_fwd, which the pages
 * describe only in its forward direction.  bf16 products with float32
 * accumulation; P and dS are rounded to bf16 (nearest even) before the
 * products they feed.  Alignment: pointers to bf16 tensors 16-byte aligned,
 * lse and delta 4-byte aligned.  dq, dk, dv and delta must not overlap each
 * other or any input.  Errors: as for fa_fwd.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int S, int D, int causal, float scale, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as fa_bwd without the delta
 * buffer: Delta lives in a fixed device array of the library (8 MiB per GPU,
 * held until the process ends), so the call allocates nothing and only
 * enqueues the same kernels.  B*H*S must be at most FA_BWD_SCRATCH_ROWS, else
 * FA_ERR_SCRATCH (nothing enqueued).  The first call on a GPU looks up the
 * array's address there (FA_ERR_LAUNCH if that fails).  All calls on one GPU
 * share its array: calls that overlap in time on one GPU (different streams
 * without ordering between them) race on it and give wrong results; calls
 * ordered on one stream are safe.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int S, int D, int causal, float scale, void* stream);

/*
 * fa_fwd_plan -- the launch shape fa_fwd (elem_bytes = 2) or fa_fwd_f32
 * (elem_bytes = 4) uses for this problem, computed on the host without any
 * HIP call (callable without a GPU).  One workgroup processes one tile of
 * query rows of one (batch, head) -- the FlashAttention-2 blog's split of the
 * work over sequence length ("FlashAttention-2 Optimizations", parallelism).
 *   rows_per_group : query rows per workgroup
 *   keys_per_tile  : keys per K/V tile staged in on-chip memory
 *   threads        : threads per workgroup (64 per wavefront; a wavefront
 *                    owns 32 query rows, at D = 256 in bf16 a pair of them)
 *   groups         : workgroups in the grid
 * A single query row (S = 1 here, Sq = 1 for fa_fwd_kv) of at most 256
 * (batch, head) pairs with D <= 128 in bf16 runs the decode kernel instead:
 * rows_per_group = 1, keys_per_tile = 2048 / D keys read per block into
 * registers (not staged), threads = 512, groups = B * H.
 * For fa_fwd_kv use fa_fwd_kv_plan (with the causal mask the choice also
 * depends on the key count).  Outputs are host pointers; each may be NULL.
 * Returns FA_ERR_SHAPE, FA_ERR_HEADDIM or FA_ERR_CAUSAL where fa_fwd would
 * (FA_ERR_SHAPE also for elem_bytes other than 2 or 4), leaving the outputs
 * untouched; else FA_OK.
 */
int fa_fwd_plan(int B, int H, int S, int D, int causal, int elem_bytes,
                int* rows_per_group, int* keys_per_tile, int* threads, int* groups);

/*
 * fa_fwd_kv_plan -- the launch shape fa_fwd_kv uses for Sq queries against
 * Sk keys (bf16), computed on the host without any HIP call; outputs as for
 * fa_fwd_plan.  Queries behind a key prefix at least as long as themselves
 * have work-balanced query tiles, which changes the workgroup choice.
 * Returns the status fa_fwd_kv would return for these sizes, leaving the
 * outputs untouched on error; else FA_OK.
 */
int fa_fwd_kv_plan(int B, int H, int Sq, int Sk, int D, int causal,
                   int* rows_per_group, int* keys_per_tile, int* threads, int* groups);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_str(int status);

/* ABI version of this library; bumped on any incompatible change. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
