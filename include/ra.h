/*
 * ra.h -- C ABI of the exact blockwise ring-attention library for MI355X (gfx950).
 *
 * What the library computes (sources are the pages, cited by title/section):
 *
 *  - Blockwise attention: one query block attended against one key/value block
 *    gives a partial output block_out and its natural-log row log-sum-exp
 *    block_lse ("flash-attention kernel that computes the next block";
 *    TokenRing review, pith.science, "What carries the argument" and "Core
 *    claim"; Ring Attention record, anthology-of-the-sota, the paragraph on
 *    blockwise attention over a ring of devices).
 *  - The merge rule that folds a partial into the running pair (TokenRing
 *    review, "What carries the argument"; paper section 3.1):
 *        out <- out - sigmoid(block_lse - lse) * (out - block_out)
 *        lse <- lse - ln sigmoid(lse - block_lse)
 *    Both right-hand sides use the old lse.  The result is exact softmax
 *    attention (Ring Attention record: no approximation).
 *  - The P-step ring schedule emulated on one GPU as a sequence of block
 *    steps in device memory: Ring Attention's K/V rotation (each rank sees K/V
 *    ranks r, r-1, ... mod P) or TokenRing's order (the owner of Q_r receives
 *    partials from K/V ranks r, r+1, ... mod P; review's Algorithm 1 comment,
 *    paper section 3.2), with the zigzag causal partition (review, "If this is
 *    right" and the section 3.3.2 comment): 2P chunks, rank r holds chunks r
 *    and 2P-1-r.  Fully masked (query chunk, key chunk) pairs are skipped.
 *
 * Conventions shared by every call:
 *  - Tensors are described by ra_tensor: a DEVICE pointer owned by the caller,
 *    sizes (b, s, h, d) and element strides (sb, ss, sh); the last dimension d
 *    has stride 1.  Q, K, V are [B, S, H, d] ("BSHD").  out / block_out are
 *    fp32 [B, S, Hq, d].  lse / block_lse are fp32 with d = 1 and logical
 *    shape [B, S, Hq]; the usual memory layout is [B, Hq, S] (sb = Hq*S,
 *    sh = S, ss = 1), but any strides are accepted.
 *  - Softmax scale is 1/sqrt(d).  lse is a natural logarithm of the sum of
 *    exp(scaled scores).  A query row that sees no key has out = 0 and
 *    lse = -inf (the merge rule's identity).
 *  - Grouped / multi-query attention: query head h reads K/V head
 *    floor(h / (Hq / Hkv)); Hq must be a multiple of Hkv.
 *  - bf16 inputs are multiplied on the matrix cores with fp32 accumulation;
 *    the softmax probabilities are rounded to bf16 (round to nearest even)
 *    before the P*V product.  fp32 inputs are computed in fp32 throughout.
 *  - Supported head_dim: 64 and 128.  Sizes up to 2^31-1 tokens per sequence;
 *    head strides (sh) up to 2^31-1 elements; bf16 K/V token strides (ss) up
 *    to (2^31-1-d)/31 elements (about 69 million); B * Hq * (Sq / 128 + 1024)
 *    below 2^31 (one launch counts its work tiles in 32 bits).  Beyond these:
 *    RA_E_UNSUPPORTED.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *    asynchronous on that stream; device faults surface at the caller's next
 *    synchronisation.
 *  - Errors: on any status other than RA_OK nothing has been enqueued and no
 *    output has been touched.  Argument checks are pure host code and run
 *    before any HIP runtime call, so they work on a machine with no GPU.
 *    ra_last_error() returns a thread-local message for the last failure.
 *    No C++ exception crosses this interface.
 *  - Ownership: the library never allocates or frees caller memory.  Scratch
 *    (partials of the unfused merge path, split-K partials) comes from the
 *    caller's workspace; its size is given by the *_workspace_bytes queries.
 *  - Results are bitwise deterministic run to run (no atomics).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RA_VERSION 1

typedef enum ra_status {
  RA_OK = 0,
  RA_E_INVALID = 1,      /* bad argument: null pointer, size or shape mismatch */
  RA_E_UNSUPPORTED = 2,  /* valid but not supported: dtype, head_dim, layout */
  RA_E_ALIGN = 3,        /* pointer or stride not aligned to 16 bytes / d not contiguous */
  RA_E_HIP = 4,          /* a HIP runtime call failed (see ra_last_error) */
  RA_E_WORKSPACE = 5     /* workspace missing or smaller than required */
} ra_status;

typedef enum ra_dtype { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

/* Mask kinds of ra_block_attn_fwd.  Query row i, key row j (0-based, local):
 *   NONE:               every key visible
 *   CAUSAL:             key j visible iff j <= i           (diagonal block)
 *   CAUSAL_BOTTOM_RIGHT key j visible iff j <= i + Sk - Sq (queries are the
 *                       last Sq positions of the key sequence; decode style) */
typedef enum ra_mask {
  RA_MASK_NONE = 0,
  RA_MASK_CAUSAL = 1,
  RA_MASK_CAUSAL_BOTTOM_RIGHT = 2
} ra_mask;

typedef struct ra_tensor {
  void *data;          /* device pointer, 16-byte aligned (4-byte for lse)   */
  int32_t dtype;       /* ra_dtype                                            */
  int32_t reserved;
  int64_t b, s, h, d;  /* sizes: batch, tokens, heads, head_dim (d=1 for lse) */
  int64_t sb, ss, sh;  /* element strides of batch, token, head              */
} ra_tensor;

/* Ring layouts of ra_ring_forward.  All tensors stay in natural token order;
 * ranks' shares are row ranges (views), never copies.
 *   CONTIG:          rank r owns tokens [r S/P, (r+1) S/P); non-causal.
 *   CONTIG_CAUSAL:   same partition, causal mask on global positions; K/V
 *                    ranks after the owner are skipped.
 *   ZIGZAG_CAUSAL:   2P chunks of S/(2P); rank r owns chunks r and 2P-1-r;
 *                    causal mask on global positions; fully masked chunk
 *                    pairs skipped.
 *   KV_SHARDED:      queries are not partitioned (one owner, e.g. a decode
 *                    step with Sq != Sk); K/V is cut into P contiguous blocks,
 *                    each visited once; non-causal.
 *   KV_SHARDED_CAUSAL: as KV_SHARDED, but the queries are the last Sq of the
 *                    Sk tokens (query i sits at position Sk - Sq + i: a prefill
 *                    chunk or decode step against a sharded cache) and the
 *                    causal mask applies on those positions (bottom-right
 *                    aligned).  Needs Sq <= Sk.  Block 0 is visible to every
 *                    query, so each row has a partial from the first step.
 *                    (TokenRing review, "Reading between the lines": the
 *                    decode / chunked-prefill extension with K/V kept in place
 *                    and partials returned to the query owner.) */
typedef enum ra_layout_kind {
  RA_LAYOUT_CONTIG = 0,
  RA_LAYOUT_CONTIG_CAUSAL = 1,
  RA_LAYOUT_ZIGZAG_CAUSAL = 2,
  RA_LAYOUT_KV_SHARDED = 3,
  RA_LAYOUT_KV_SHARDED_CAUSAL = 4
} ra_layout_kind;

/* Merge order of the emulated ring.
 *   RING:      step t merges K/V rank (r - t) mod P (Ring Attention).
 *   TOKENRING: step t merges K/V rank (r + t) mod P (TokenRing: the owner
 *              receives the partial computed on rank r + t). */
typedef enum ra_order { RA_ORDER_RING = 0, RA_ORDER_TOKENRING = 1 } ra_order;

typedef struct ra_layout {
  int32_t kind;            /* ra_layout_kind                                    */
  int32_t order;           /* ra_order                                          */
  int32_t rank;            /* -1: emulate every rank; r >= 0: rank r's rows only */
  int32_t fuse_merge;      /* 1: merge inside the attention epilogue (no
                              block_out round trip); 0: attention writes
                              block_out/block_lse to the workspace and a separate
                              merge kernel folds them in                        */
  void *workspace;         /* device scratch owned by the caller (may be NULL
                              when ra_ring_workspace_bytes returns 0)            */
  size_t workspace_bytes;
} ra_layout;

/* One work item of the ring plan: a run of query rows of one owner rank
 * against up to two key segments, in one step.  Positions are natural token
 * indices.  Items of one step write disjoint query rows. */
typedef struct ra_plan_seg {
  int64_t kv_start, kv_len;  /* key rows [kv_start, kv_start + kv_len)        */
  int32_t causal;            /* 1: key visible iff its position <= query's    */
  int32_t kv_rank;           /* rank that holds these keys                    */
} ra_plan_seg;

typedef struct ra_plan_item {
  int32_t step;              /* 0 .. P-1                                       */
  int32_t rank;              /* owner of the query rows                        */
  int64_t q_start, q_len;    /* query rows [q_start, q_start + q_len)          */
  int32_t nseg;              /* 1 or 2                                         */
  int32_t first;             /* 1: first partial for these rows (overwrites)   */
  ra_plan_seg seg[2];
  int64_t q_pos0;            /* token position of row q_start (= q_start except
                                for KV_SHARDED_CAUSAL: q_start + Sk - Sq)      */
} ra_plan_item;

/* ra_block_attn_fwd -- block_out, block_lse of one query block against one
 * key/value block (TokenRing review, "What carries the argument": the
 * flash-attention kernel computing a block).
 *   q:   [B, Sq, Hq, d]  bf16 or fp32                      (read)
 *   k,v: [B, Sk, Hkv, d] same dtype as q                   (read)
 *   causal_mask_kind: ra_mask
 *   out: [B, Sq, Hq, d] fp32                               (written: block_out)
 *   lse: [B, Sq, Hq] fp32 (d = 1; usually stored [B, Hq, Sq]) (written: block_lse)
 * Sk may be 0 (then out = 0, lse = -inf).  Sq may be 0 (nothing enqueued).
 * When Sq * (Hq/Hkv) is small (decode) the keys are split over work-groups;
 * the split partials then need workspace from ra_block_attn_workspace_bytes
 * (passing workspace = NULL disables the split: same result, slower). */
ra_status ra_block_attn_fwd(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                            int causal_mask_kind, ra_tensor *out, ra_tensor *lse,
                            void *workspace, size_t workspace_bytes, void *stream);

size_t ra_block_attn_workspace_bytes(const ra_tensor *q, const ra_tensor *k);

/* ra_block_attn_fwd_noalloc -- ra_block_attn_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, same kernels and same
 * results as ra_block_attn_fwd with a workspace of
 * ra_block_attn_workspace_bytes(q, k) bytes, but the split-K partials live in
 * a static device array of RA_NOALLOC_SCRATCH_BYTES held by the library: one
 * copy per GPU, allocated when the code object is loaded and kept until the
 * process ends.  No call allocates or frees memory.
 *   - A block whose split partials need more than RA_NOALLOC_SCRATCH_BYTES
 *     (ra_block_attn_workspace_bytes > the limit) is rejected with
 *     RA_E_UNSUPPORTED before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two host threads) race and give wrong
 *     results.  Calls in one stream are ordered and safe.  The array keeps the
 *     last call's partials; nothing in it needs to start at zero (every
 *     partial is written before it is read).
 *   - The first call on a device (with that device current) looks up the
 *     array's device address; a failure there is RA_E_HIP. */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

ra_status ra_block_attn_fwd_noalloc(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v,
                                    int causal_mask_kind, ra_tensor *out, ra_tensor *lse,
                                    void *stream);

/* ra_merge -- fold a partial into the running pair, in place (TokenRing
 * review, "What carries the argument"; paper section 3.1).
 *   out, block_out: [B, S, H, d] fp32;  lse, block_lse: [B, S, H] fp32 (d = 1).
 *   d is one of 4, 8, 16, 32, 64, 128, 256 (else RA_E_UNSUPPORTED).
 * out/lse are read and overwritten; block_* are read.  An lse of -inf is the
 * identity on either side.  out must not alias block_out. */
ra_status ra_merge(ra_tensor *out, ra_tensor *lse, const ra_tensor *block_out,
                   const ra_tensor *block_lse, void *stream);

/* ra_ring_forward -- exact attention of the full sequence through the
 * emulated P-step ring (Ring Attention record; TokenRing review, "Core
 * claim" and section 3.2).
 *   q: [B, Sq, Hq, d], k, v: [B, Sk, Hkv, d] in natural token order.
 *   out: [B, Sq, Hq, d] fp32, lse: [B, Sq, Hq] fp32 (d = 1).
 * For every layout except KV_SHARDED, Sq == Sk and S % P == 0 (CONTIG*) or
 * S % 2P == 0 (ZIGZAG).  Rows owned by the emulated rank(s) are written
 * (initialised by the first step, then merged step by step); other rows are
 * untouched.  1 <= P <= 16.
 * KV_SHARDED with fuse_merge = 1, when one block's query tiles cannot fill
 * the chip (decode): the P blocks' partials do not depend on each other, so
 * all of them run in one launch, each block cut into sub-blocks, and one
 * reduction combines every partial into (out, lse) in closed form -- the
 * gather-merge of the ranks' partials, equal to folding them with the merge
 * rule in plan order up to rounding.  The workspace then holds the partials
 * (ra_ring_workspace_bytes). */
ra_status ra_ring_forward(const ra_tensor *q, const ra_tensor *k, const ra_tensor *v, int P,
                          const ra_layout *layout, ra_tensor *out, ra_tensor *lse,
                          void *stream);

/* Bytes of workspace ra_ring_forward needs for these shapes: block results
 * when unfused, split-K partials for KV_SHARDED decode shapes, else 0. */
size_t ra_ring_workspace_bytes(const ra_tensor *q, const ra_tensor *k, int P,
                               const ra_layout *layout);

/* ra_ring_plan -- the host-only work list (no HIP call).  Writes up to
 * max_items items in step order (items may be NULL to query the count) and
 * returns the number of items, or -1 on invalid arguments. */
int ra_ring_plan(int64_t Sq, int64_t Sk, int P, const ra_layout *layout,
                 ra_plan_item *items, int max_items);

/* Per-kernel timing with HIP events on the caller's stream (instrumentation,
 * off by default).  ra_profile_enable(1) clears the counters and records an
 * event pair around every kernel launch; ra_profile_read() synchronises on
 * those events and returns, for each kernel kind, its launch count and the
 * summed device time in milliseconds. */
typedef enum ra_kernel_kind {
  RA_KERNEL_ATTN = 0,        /* attention (with or without fused merge)  */
  RA_KERNEL_MERGE = 1,       /* standalone merge                          */
  RA_KERNEL_SPLIT_REDUCE = 2,/* split-K reduction (decode shapes)         */
  RA_KERNEL_KIND_COUNT = 3
} ra_kernel_kind;

ra_status ra_profile_enable(int on);
ra_status ra_profile_read(int64_t *launches, double *total_ms, int n_kinds);

const char *ra_status_str(int status);
const char *ra_last_error(void);
int ra_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
