/*
 * attn.h -- C ABI of libattn.so: fused attention forward (prefill), KV-cache
 * decode and the KV-cache writer, hand-written HIP kernels for MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [P1] "Skill: Write a Triton Attention Kernel"
 *   [P2] "FlashAttention Kernel Optimization" (flash-attention-kernel skill)
 *   [P3] "Triton-FlashAttention" (project README)
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory and keeps no mutable global state.
 *   - Strides are in ELEMENTS (not bytes), 64-bit, one per logical dimension,
 *     so any (B,H,N,D) or (B,N,H,D) view is accepted ([P1] "Inputs" item 7 and
 *     "Kernel design rules": all strides are arguments, no contiguity assumed).
 *     The innermost (head-dim) stride must be 1, every other stride a multiple
 *     of 8 elements, and every base pointer 16-byte aligned: the kernels move
 *     rows in 16-byte vectors.  Row (sequence / cache slot) strides are at
 *     most 2^22 elements: a tile's rows are addressed with 32-bit offsets from
 *     its first row (base and row offsets themselves are 64-bit, so tensors
 *     and offsets beyond 2^31 bytes are fine).  Output views (o, dq, dk, dv,
 *     the caches and page pools written) must address every element once:
 *     ordered by stride, each dimension of extent > 1 steps past the whole
 *     span of the smaller ones (heads or rows that alias would have several
 *     workgroups race on one address).  Violations return
 *     ATTN_ERR_UNSUPPORTED.
 *   - Element types: IEEE fp16 or bf16 for Q/K/V/O; scores, softmax state and
 *     accumulators are fp32 inside the kernels ([P1] "Kernel design rules").
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream).  Every
 *     call is asynchronous on that stream; the caller synchronises.
 *   - Every argument is validated on the host before anything is enqueued.  On
 *     any error nothing is launched and no memory is touched ([P3] GQA phase:
 *     unsupported cases must refuse rather than run silently).  Errors are
 *     returned, never thrown.
 *   - Causal and band prefill calls (attn_fwd, attn_fwd_masked and their
 *     packed forms) whose blocks run 256 rows coordinate the waves of a block
 *     through counters in LDS, with bounded waits.  A correct run never
 *     reaches the bound; if a wait ever ran out, that block writes NaN to all
 *     of its o rows and lse entries instead of values it could not trust.  The
 *     environment variable ATTN_RING_POLL_LIMIT (read on every call, clamped
 *     to [1, 2^18], default 2^18) lowers the bound, for tests of that path.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                          */
  ATTN_ERR_SHAPE = 2,       /* a size <= 0, Hq % Hkv != 0, cache_len or pos range  */
  ATTN_ERR_UNSUPPORTED = 3, /* D not in {64,128}, unknown dtype, stride/alignment  */
  ATTN_ERR_WORKSPACE = 4,   /* decode workspace missing or smaller than required   */
  ATTN_ERR_HIP = 5          /* the HIP runtime reported an error at launch         */
} attn_status;

/* Element strides of a 4-D tensor viewed as (batch, head, position, head_dim). */
typedef struct {
  int64_t b, h, n, d;
} attn_strides;

/* causal argument of attn_fwd */
enum {
  ATTN_CAUSAL_NONE = 0,         /* every key j < Nkv is visible */
  ATTN_CAUSAL_TOP_LEFT = 1,     /* j <= i: the pages' mask ([P1] step 5c) */
  ATTN_CAUSAL_BOTTOM_RIGHT = 2  /* j <= i + (Nkv - Nq): the Nq queries are the last
                                   Nq positions of the Nkv-token sequence (chunked
                                   prefill, multi-token verification) */
};

/* alignment of a mask's diagonal: query i sits at key position p = i + off */
enum {
  ATTN_ALIGN_TOP_LEFT = 0,     /* off = 0 */
  ATTN_ALIGN_BOTTOM_RIGHT = 1  /* off = Nkv - Nq (per sequence for packed batches) */
};

/*
 * A band mask around each query's position p: key j is visible iff
 * p - window_left <= j <= p + window_right (and j < Nkv); -1 leaves a side
 * open.  {align, -1, 0} is the causal mask ([P1] step 5c with align top-left),
 * {align, -1, -1} no mask, {align, w - 1, 0} a causal sliding window of w keys
 * ([P1] "Use this when": windowed attention; [P3] deferred scope).
 * A side of max(Nq, Nkv) or more (packed batches: max(total_q, total_k))
 * hides no key and is treated as open, INT32_MAX included.  A mask that is
 * still a band after that (neither unmasked nor causal) needs Nq, Nkv (packed:
 * total_q, total_k) <= 2^28; longer sequences give ATTN_ERR_UNSUPPORTED.
 */
typedef struct {
  int32_t align;         /* ATTN_ALIGN_TOP_LEFT or ATTN_ALIGN_BOTTOM_RIGHT */
  int32_t window_left;   /* >= -1 */
  int32_t window_right;  /* >= -1 */
} attn_mask;

/*
 * attn_fwd -- O = softmax(scale * Q K^T + mask) V, one fused kernel.
 *
 * Defines: [P1] "Required reasoning process" steps 1-9 (tiling over KV blocks,
 * online softmax with running max m and running sum l, alpha rescale, P.V
 * accumulation, final 1/l, logsumexp, causal loop end); [P2] "Online Softmax",
 * "Tiled Computation", "Causal Masking"; [P3] GQA design (kv_head = q_head /
 * group).
 *
 *   q    (B, Hq,  Nq,  D) via sq      k, v (B, Hkv, Nkv, D) via sk, sv
 *   o    (B, Hq,  Nq,  D) via so      written, same dtype as q
 *   lse  nullable; if given, contiguous fp32 (B, Hq, Nq):
 *        lse[b,h,i] = ln sum_{visible j} exp(scale * q_i . k_j)   ([P1] step 8)
 *   Hq % Hkv == 0; q head h reads kv head h / (Hq / Hkv).
 *   causal: ATTN_CAUSAL_NONE, ATTN_CAUSAL_TOP_LEFT (key j visible to query i
 *        iff j <= i, [P1] step 5c) or ATTN_CAUSAL_BOTTOM_RIGHT (j <= i + Nkv - Nq;
 *        with Nq > Nkv the first Nq - Nkv rows see no key and get o = 0 and
 *        lse = -inf); other values give ATTN_ERR_UNSUPPORTED.  Blocks wholly
 *        above the diagonal are never visited.
 *   scale: multiplies the fp32 scores (any finite value, 0 and negative
 *        included; the caller typically passes 1/sqrt(D)).
 *   D in {64, 128}.  Nq, Nkv >= 1, any value (ragged tails are masked).
 *   Rows of o beyond Nq and elements outside the described views are never
 *   written; K/V rows at positions >= Nkv are never read.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                     float scale, int causal, attn_dtype dtype, void* stream);

/*
 * attn_fwd_masked -- attn_fwd with a band mask (attn_mask) in place of the
 * causal argument.  Tiles wholly outside the band of a block's rows are never
 * visited on either side.  Rows that see no key get o = 0 and lse = -inf.
 * Other arguments, layouts and errors as attn_fwd; an align outside the enum
 * or a window bound below -1 gives ATTN_ERR_UNSUPPORTED.
 */
attn_status attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                            attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            float scale, attn_mask mask, attn_dtype dtype, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over a batch of packed sequences of different
 * lengths: sequence b owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and
 * key/value rows [cu_seqlens_k[b], cu_seqlens_k[b+1]) of the packed tensors,
 * and attends only to its own keys.  Within a sequence the operation is that of
 * attn_fwd ([P1] "Required reasoning process" steps 1-9, [P2] "Online
 * Softmax", [P3] GQA design); the packed variable-length batch itself is the
 * widening that [P3]'s deferred scope names (varlen).
 *
 *   q    (total_q, Hq,  D): row t of head h at q[t*sq.n + h*sq.h + d]  (sq.b unused)
 *   k, v (total_k, Hkv, D) via sk, sv (b unused)
 *   o    (total_q, Hq,  D) via so (b unused); written, same dtype as q
 *   lse  nullable; if given, contiguous fp32 (Hq, total_q): lse[h*total_q + t]
 *   cu_seqlens_q, cu_seqlens_k: DEVICE int32 arrays of B + 1 offsets, expected
 *        non-decreasing from 0 to total_q (total_k).  They are read on the GPU
 *        (no host synchronisation); each offset is clamped into [previous
 *        offset, total], so malformed offsets give empty or shortened sequences
 *        but never an access outside the packed tensors.
 *   max_seqlen_q: host bound on the query rows of any sequence; sizes the grid
 *        (ceil(max_seqlen_q/R) query blocks per (sequence, head), R = 128
 *        rows when total_q <= 6144 * B, else 256).  Query
 *        rows at positions >= max_seqlen_q within a sequence are not computed
 *        and their o rows and lse entries are left untouched; the mask of the
 *        rows computed is still that of the whole sequence.
 *   causal: as attn_fwd, per sequence: ATTN_CAUSAL_TOP_LEFT (j <= i) or
 *        ATTN_CAUSAL_BOTTOM_RIGHT (j <= i + L_k - L_q with the sequence's own
 *        lengths).  A row with no visible key (a sequence with L_k = 0, or the
 *        first L_q - L_k rows bottom-right) gets o = 0 and lse = -inf.
 *   B >= 1, max_seqlen_q >= 1, total_q >= 1, total_k >= 0; D in {64, 128};
 *   strides, alignment and dtype rules as attn_fwd; the offset arrays must be
 *   4-byte aligned.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B, int max_seqlen_q,
                            int total_q, int total_k, int Hq, int Hkv, int D,
                            attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            float scale, int causal, attn_dtype dtype, void* stream);

/*
 * attn_fwd_varlen_masked -- attn_fwd_varlen with a band mask (attn_mask); the
 * diagonal of each sequence follows mask.align with that sequence's own
 * lengths.  Otherwise as attn_fwd_varlen and attn_fwd_masked.
 */
attn_status attn_fwd_varlen_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int B,
                                   int max_seqlen_q, int total_q, int total_k, int Hq, int Hkv, int D,
                                   attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                                   float scale, attn_mask mask, attn_dtype dtype, void* stream);

/*
 * attn_bwd_workspace_bytes -- scratch attn_bwd needs: B * Hq * Nq * 8 bytes
 * (one (lse * log2 e, delta) pair of floats per query row).  0 for invalid sizes.
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/*
 * attn_bwd -- gradients of attn_fwd's O with respect to Q, K and V for an
 * upstream gradient dO: the backward the pages name as a separate, later
 * kernel pair that recomputes the attention weights from the forward's
 * logsumexp ([P1] "Do not use this when" and "Correctness requirements",
 * lse bullet; [P3] Phase 1: separate dq and dk/dv kernels with masked loads;
 * [P3] deferred scope: GQA backward accumulates every q head of a group into
 * the shared dK, dV).
 *
 *   P  = exp(scale q_i . k_j - lse_i) on visible (i, j), else 0
 *   dV = P^T dO;  dP = dO V^T;  dS = P (dP - delta_i), delta_i = sum_d dO_i,d O_i,d
 *   dQ = scale dS K;  dK = scale dS^T Q;  a kv head's dK, dV sum its group's q heads
 *
 *   q, o, dout, dq (B, Hq, Nq, D) and k, v, dk, dv (B, Hkv, Nkv, D) via their
 *   strides (rules as attn_fwd); dq, dk, dv are written (same dtype as q).
 *   lse: contiguous fp32 (B, Hq, Nq), as attn_fwd returns it for the same
 *   inputs, causal argument and scale.  causal: as attn_fwd (attn_bwd_masked
 *   takes a band mask).  workspace: attn_bwd_workspace_bytes(B, Hq, Nq)
 *   bytes, 16-byte aligned, contents irrelevant.  Two kernels run in order on
 *   `stream`: dQ (which also leaves each query row's statistics in the
 *   workspace), then dK/dV; no atomics, so the result does not depend on
 *   scheduling.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                     attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so, attn_strides sdo,
                     attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale, int causal,
                     attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_masked -- attn_bwd with a band mask (attn_mask) in place of the
 * causal argument, the backward of attn_fwd_masked with the same mask: the
 * dQ pass visits only the key tiles inside its rows' band and the dK/dV pass
 * only the query tiles whose band reaches its keys.  Otherwise as attn_bwd.
 */
attn_status attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nkv,
                            int D, attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                            attn_strides sdo, attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale,
                            attn_mask mask, attn_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd_varlen, attn_bwd_varlen_masked -- the backward of attn_fwd_varlen
 * (attn_fwd_varlen_masked): attn_bwd on each packed sequence's own rows; no
 * gradient crosses sequences.  Layouts, offsets (clamped on the device) and
 * the per-sequence mask as the packed forward: q, o, dout, dq (total_q, Hq, D),
 * k, v, dk, dv (total_k, Hkv, D) via strides (b unused); lse contiguous fp32
 * (Hq, total_q) as attn_fwd_varlen returns it.  max_seqlen_q, max_seqlen_k:
 * host bounds on every sequence's query and key rows (they size the grids);
 * query rows past max_seqlen_q, which the forward does not compute, are
 * ignored here too (no dq written, no contribution to dk, dv); max_seqlen_k
 * must bound every key count (dk, dv rows past it are not written).  dq rows of a
 * sequence with no keys and dk, dv rows of one with no queries are written as
 * 0.  workspace: attn_bwd_workspace_bytes(1, Hq, total_q) bytes.
 */
attn_status attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k, int total_q,
                            int total_k, int Hq, int Hkv, int D, attn_strides sq, attn_strides sk, attn_strides sv,
                            attn_strides so, attn_strides sdo, attn_strides sdq, attn_strides sdk, attn_strides sdv,
                            float scale, int causal, attn_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream);
attn_status attn_bwd_varlen_masked(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int B, int max_seqlen_q, int max_seqlen_k,
                                   int total_q, int total_k, int Hq, int Hkv, int D, attn_strides sq,
                                   attn_strides sk, attn_strides sv, attn_strides so, attn_strides sdo,
                                   attn_strides sdq, attn_strides sdk, attn_strides sdv, float scale,
                                   attn_mask mask, attn_dtype dtype, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * attn_decode_workspace_bytes -- size of the scratch buffer attn_decode needs
 * for a cache of S_max slots (covers every cache_len <= S_max and every split
 * count): U * min(64, ceil(S_max/128)) * ceil(G/ceil(G/16)) * (D + 4) * 4
 * bytes, with G = Hq / Hkv and U = B * Hkv * ceil(G/16) (batch, kv head, head
 * group) slots.  Returns 0 for invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int S_max, int D);

/*
 * attn_decode -- one query token per (batch, q head) attending to cache slots
 * [0, cache_len) of a preallocated KV cache ([P3] decode phase: separate decode
 * kernel, cache_len is a runtime value, GQA indexing as in prefill, every
 * cached position visible).  The cache is split along its length into chunks
 * processed in parallel; each chunk's (max, sum, unnormalised output) partial
 * is merged by a second kernel with the same rescale identity the online
 * softmax uses ([P1] step 5f, [P2] "Online Softmax").
 *
 *   q        (B, Hq, D): element (b,h,d) at q[b*sq.b + h*sq.h + d]  (sq.n unused)
 *   k_cache, v_cache (B, Hkv, S_max, D) via skc, svc
 *   o        (B, Hq, D) via so (so.n unused);  lse nullable, contiguous fp32 (B, Hq)
 *   1 <= cache_len <= S_max.  Slots >= cache_len are never read.
 *   num_splits: 0 = library heuristic; k > 0 asks for k chunks (clamped to
 *               [1, 64] and to the number of 128-slot tiles) -- used to test
 *               that the result does not depend on the split.
 *   workspace: device scratch of at least attn_decode_workspace_bytes(...)
 *              bytes, 16-byte aligned, contents irrelevant (no initialisation
 *              needed).  Calls that may run concurrently (different streams)
 *              need distinct workspaces.
 */
attn_status attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                        int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                        attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                        float scale, attn_dtype dtype, int num_splits,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, allocation-free serving loops,
 * harnesses that forbid hipMalloc): the same kernels, with the split partials
 * kept in a fixed scratch array inside the library instead of a caller's
 * workspace.  No allocation happens in this call or in the library.
 *
 *   Arguments, layouts, results and errors as attn_decode (no workspace).
 *   Scratch: ATTN_DECODE_NOALLOC_SCRATCH_BYTES per GPU, in the library's device
 *   memory, held until the process ends.  A call whose partials, B * Hkv *
 *   ceil(G/16) * n * ceil(G/ceil(G/16)) * (D + 4) * 4 bytes for its n > 1
 *   chunks (G = Hq / Hkv; none when n = 1), exceed it returns
 *   ATTN_ERR_WORKSPACE and launches nothing.  At the default split count
 *   (num_splits = 0: fewer than 1024 chunks in all) the partials stay below
 *   8.7 MB and always fit; only a forced num_splits can exceed the scratch.
 *   Every call on a GPU shares that GPU's scratch: calls that may overlap on
 *   one GPU (different streams, or host threads) race and must be serialised
 *   by the caller.  The first call on a device looks up the scratch's address
 *   there (with that device current) and keeps it.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                                int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                                attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                                float scale, attn_dtype dtype, int num_splits, void* stream);

/*
 * attn_decode_varlen -- attn_decode with a length per sequence: batch element
 * b attends to its cache slots [0, cache_lens[b]).  Per-sequence lengths are
 * the first item of [P3]'s deferred scope ("Out of scope for now": decode for
 * sequences of different lengths in one batch); everything else is
 * attn_decode's definition.
 *
 *   cache_lens     device pointer to B int32 values, 4-byte aligned; each is
 *                  used as min(max(cache_lens[b], 0), max_cache_len).  A
 *                  sequence of length 0 gets o = 0 and lse = -inf.
 *   max_cache_len  host bound, 1 <= max_cache_len <= S_max; it sizes the
 *                  split grid (passing S_max is always valid; a tighter bound
 *                  launches fewer empty chunks).  Slots at or beyond a
 *                  sequence's length are never read.
 *   Other arguments, the workspace rules and the error codes are attn_decode's;
 *   a null cache_lens gives ATTN_ERR_NULL.
 */
attn_status attn_decode_varlen(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                               int B, int Hq, int Hkv, int S_max, const int32_t* cache_lens, int max_cache_len,
                               int D, attn_strides sq, attn_strides skc, attn_strides svc, attn_strides so,
                               float scale, attn_dtype dtype, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged -- attn_decode_varlen over a paged KV cache: cache slot r
 * of sequence b lives in page block_table[b * max_pages_per_seq + r / page_size],
 * row r % page_size, of the page pools.  The paged cache is the widening that
 * [P3]'s deferred scope names; per sequence the operation is the decode of
 * [P3] decode phase over that sequence's first cache_lens[b] slots.
 *
 *   q        (B, Hq, D) via sq (sq.n unused);  o (B, Hq, D) via so (so.n unused)
 *   k_pages, v_pages: page pools (num_pages, Hkv, page_size, D) via skp, svp:
 *            element (p, h, r, d) at k_pages[p*skp.b + h*skp.h + r*skp.n + d]
 *            (so (num_pages, page_size, Hkv, D) pools are accepted too)
 *   block_table: DEVICE int32 (B, max_pages_per_seq), row-major; page ids are
 *            clamped into [0, num_pages) on the device
 *   cache_lens: DEVICE int32 (B), clamped to [0, max_cache_len]; a length of 0
 *            gives o = 0 and lse = -inf
 *   page_size: a power of two, 16 <= page_size <= 2^20 (else UNSUPPORTED)
 *   max_cache_len: host bound on the lengths, <= max_pages_per_seq * page_size;
 *            sizes the split grid
 *   lse nullable, contiguous fp32 (B, Hq); num_splits as attn_decode
 *   workspace: attn_decode_workspace_bytes(B, Hq, Hkv, max_cache_len, D) bytes
 *   Only the pages a sequence's first cache_lens[b] slots map to are read.
 */
attn_status attn_decode_paged(const void* q, const void* k_pages, const void* v_pages, void* o, float* lse,
                              int B, int Hq, int Hkv, int num_pages, int page_size,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* cache_lens, int max_cache_len, int D,
                              attn_strides sq, attn_strides skp, attn_strides svp, attn_strides so,
                              float scale, attn_dtype dtype, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Options of attn_decode_ex: which cache form, and an optional sliding window. */
typedef struct {
  const int32_t* cache_lens;   /* DEVICE int32 (B), or NULL: every sequence has cache_len slots */
  const int32_t* block_table;  /* DEVICE int32 (B, max_pages_per_seq), or NULL: contiguous caches */
  int32_t max_pages_per_seq;   /* paged caches only */
  int32_t page_size;           /* paged caches only: a power of two, 16 .. 2^20 */
  int32_t num_pages;           /* paged caches only */
  int32_t window_left;         /* -1: every slot; w >= 0: only slots >= len - 1 - w */
} attn_decode_opts;

/*
 * attn_decode_ex -- attn_decode, attn_decode_varlen and attn_decode_paged in
 * one entry point, with an optional sliding window ([P1] "Use this when":
 * windowed attention; [P3] deferred scope).  The query of sequence b is the
 * token in its last slot, len - 1 (as after kv_cache_write of that token), so
 * a window of w keeps the last w + 1 slots; slots before them (and, paged, the
 * block-table entries and pages that hold only such slots) are never read.
 *   cache_lens NULL, block_table NULL: as attn_decode (cache_len for all, caches
 *     (B, Hkv, S_max, D)).
 *   cache_lens set, block_table NULL: as attn_decode_varlen (cache_len is the
 *     bound max_cache_len).
 *   block_table set (cache_lens required): as attn_decode_paged (k, v are the
 *     page pools, cache_len is max_cache_len, S_max unused).
 *   workspace: attn_decode_workspace_bytes(B, Hq, Hkv, S, D) with S = S_max
 *     (contiguous) or cache_len (paged).  window_left < -1: ATTN_ERR_SHAPE.
 */
attn_status attn_decode_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int Hq, int Hkv, int S_max, int cache_len, int D,
                           attn_strides sq, attn_strides sk, attn_strides sv, attn_strides so,
                           float scale, attn_dtype dtype, int num_splits, const attn_decode_opts* opts,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_cache_write_paged -- kv_cache_write for a paged cache: row t of sequence
 * b (k_new, v_new (B, Hkv, T, D) via skn, svn) is stored at that sequence's
 * slot pos[b] + t, i.e. row (pos[b] + t) % page_size of page
 * block_table[b * max_pages_per_seq + (pos[b] + t) / page_size]  ([P3] decode
 * phase: the cache is written by a separate helper; paged per the deferred
 * scope).  pos: DEVICE int32 (B).  Slots outside [0, max_pages_per_seq *
 * page_size) are skipped and page ids are clamped into [0, num_pages) on the
 * device, so no write leaves the pools.  Pools, strides and page_size as
 * attn_decode_paged; D a multiple of 8.
 */
attn_status kv_cache_write_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                                 int B, int Hkv, int num_pages, int page_size, const int32_t* block_table,
                                 int max_pages_per_seq, const int32_t* pos, int D, int T,
                                 attn_strides skp, attn_strides svp, attn_strides skn, attn_strides svn,
                                 attn_dtype dtype, void* stream);

/*
 * kv_cache_write -- copy T new rows per (batch, kv head) into cache slots
 * [pos, pos + T) of K and V ([P3] decode phase: the preallocated-cache write
 * helper kept separate from the attention kernel).  A bit-exact copy; every
 * other cache element is untouched.
 *
 *   k_cache, v_cache (B, Hkv, S_max, D) via skc, svc
 *   k_new, v_new     (B, Hkv, T, D)     via skn, svn
 *   0 <= pos, T >= 1, pos + T <= S_max; D a positive multiple of 8.
 */
attn_status kv_cache_write(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           int B, int Hkv, int S_max, int D, int pos, int T,
                           attn_strides skc, attn_strides svc, attn_strides skn, attn_strides svn,
                           attn_dtype dtype, void* stream);

/* Static, human-readable name of a status code. */
const char* attn_status_string(attn_status s);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
