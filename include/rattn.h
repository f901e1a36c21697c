/*
 * rattn.h -- fused residual attention over a shared base KV cache (AMD Instinct
 * MI355X, gfx950).  C ABI.
 *
 * The method (ForkKV Guide, "The Copy-on-Write Paradigm" and "Fused
 * ResidualAttention"; LRAgent, "Schemi di Condivisione" and
 * "Flash-LoRA-Attention"): N LoRA agents share one base KV cache of a common
 * prefix (K_base, V_base: the bCache), and agent a keeps only rank-r residual
 * caches Lk_a, Lv_a (the rCache / "LR cache", the down-projected activations
 * X A) and the up-projections Bk_a, Bv_a, so that
 *     K_a = K_base + Lk_a Bk_a,      V_a = V_base + Lv_a Bv_a.
 * The library computes softmax(q K_a^T * scale) V_a for every agent without
 * materialising K_a or V_a, using
 *     q K_a^T = q K_base^T + (q Bk_a^T) Lk_a^T     (ForkKV Guide, "Mathematical
 *                                                   Formulation of ResidualAttention")
 *     P V_a   = P V_base + (P Lv_a) Bv_a            (LRAgent, Flash-LoRA-Attention).
 * The LoRA scale alpha/r is folded into Bk and Bv by the caller.
 *
 * Notation.  N agents; H_q query heads and H_kv KV heads (H_q % H_kv == 0);
 * query head h reads KV head floor(h / (H_q/H_kv)) (consecutive query heads share
 * a KV head); head dimension d; rank r; shared prefix length L; S private tokens
 * per agent; q_len query tokens per agent.
 *
 * Conventions for every entry point.
 *   - All tensor pointers are DEVICE pointers, owned by the caller, row-major,
 *     contiguous, and 16-byte aligned.  The library never allocates, frees or
 *     synchronises; work is enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and the call returns before it finishes.
 *   - Every argument is validated on the host before any HIP call.  A negative
 *     rattn_status is returned and nothing is launched when validation fails.
 *     A failed launch returns RATTN_E_HIP.  Faults during execution surface at
 *     the caller's next synchronisation.
 *   - Inputs are finite.  The kernels take every score to be finite or -inf (a
 *     masked key), so a NaN or infinity in q, the caches or the projections
 *     gives unspecified outputs.  Pool pages that the block table does not
 *     reference are never read and may hold anything.
 *   - Block-table entries must lie in [0, n_phys_pages); this is not checked on
 *     the device (an out-of-range entry is undefined behaviour).  Duplicate
 *     entries (aliased pages) are allowed.
 *   - The library keeps no global mutable state and is reentrant, except that
 *     rattn_last_hip_error() reports the calling thread's last HIP failure.
 */
#ifndef RATTN_H
#define RATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RATTN_VERSION 2

typedef enum rattn_status {
    RATTN_OK = 0,
    RATTN_E_NULL = -1,        /* a required pointer is NULL (or a forbidden one is not) */
    RATTN_E_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    RATTN_E_UNSUPPORTED = -3, /* valid, but outside what the kernels implement */
    RATTN_E_WORKSPACE = -4,   /* workspace NULL or smaller than rattn_workspace_bytes */
    RATTN_E_ALIGN = -5,       /* a pointer is not 16-byte aligned */
    RATTN_E_HIP = -6,         /* a HIP runtime call or kernel launch failed */
    RATTN_E_SCRATCH = -7,     /* rattn_decode_noalloc: the call needs more than its static buffer */
    RATTN_E_POOL = -8         /* page pool: not enough free pages (or host memory) */
} rattn_status;

typedef enum rattn_dtype {
    RATTN_F32 = 0, /* IEEE binary32 */
    RATTN_BF16 = 1 /* bfloat16 */
} rattn_dtype;

/* Storage of the base keys (rattn_desc.k_format). */
typedef enum rattn_key_format {
    RATTN_KEYS_DTYPE = 0, /* keys in the call's dtype, like the values */
    RATTN_KEYS_INT8 = 1   /* int8 codes with one scale per tensor (PolyKV, section 2B): byte u holds
                             code u - 128 (excess-128), key = k_scale * (u - 128); see
                             rattn_quantize_keys */
} rattn_key_format;

/* Storage of the base values (rattn_desc.v_format). */
typedef enum rattn_value_format {
    RATTN_VALUES_DTYPE = 0, /* values in the call's dtype */
    RATTN_VALUES_FWHT3 = 1  /* 3-bit codes after a Walsh-Hadamard rotation (PolyKV, section 2B,
                               TurboQuant MSE); see rattn_quantize_values for the format.  Requires
                               RATTN_KEYS_INT8 (the pages' asymmetric pairing), a contiguous base
                               cache and the same limits as int8 keys */
} rattn_value_format;

typedef enum rattn_op {
    RATTN_OP_DECODE = 0,
    RATTN_OP_PREFILL = 1,
    RATTN_OP_RECONSTRUCT = 2 /* rattn_decode_reconstruct (rattn_workspace_bytes only) */
} rattn_op;

/* Shape of one call (one layer). */
typedef struct rattn_desc {
    int32_t n_agents;     /* N >= 1 */
    int32_t n_q_heads;    /* H_q >= 1, a multiple of n_kv_heads */
    int32_t n_kv_heads;   /* H_kv >= 1 */
    int32_t head_dim;     /* d: 64 or 128 */
    int32_t rank;         /* r: 0 (no residual), 8, 16, 32, 64 or 128 */
    int32_t q_len;        /* query tokens per agent (decode: >= 1; prefill: == priv_len) */
    int64_t prefix_len;   /* L >= 0: shared base tokens */
    int64_t priv_len;     /* S >= 0: private tokens per agent; L + S >= 1 */
    int32_t page_size;    /* 0: contiguous base cache; else a multiple of 16 (paged pool) */
    int32_t shared_lr;    /* 0: per-agent Lk/Lv; 1: one Lk/Lv for all agents (BaseLRShared) */
    int64_t n_phys_pages; /* pages in the pool (paged only) */
    int32_t dtype;        /* rattn_dtype of q, caches and up-projections */
    float sm_scale;       /* softmax scale; <= 0 means 1/sqrt(head_dim) */
    int32_t k_format;     /* rattn_key_format of k_base (0: dtype).  RATTN_KEYS_INT8: bf16 decode,
                             head_dim 128, priv_len 0 (else RATTN_E_UNSUPPORTED); k_base then holds
                             one byte per element in the same layout */
    float k_scale;        /* RATTN_KEYS_INT8: the keys' scale (> 0); else ignored */
    int32_t v_format;     /* rattn_value_format of v_base (0: dtype).  RATTN_VALUES_FWHT3: v_base holds
                             [H_kv, L, 3 d / 8] bytes of codes and rattn_args.v_scale the scales */
} rattn_desc;

/* Tensors of one call.  Shapes use the descriptor's names. */
typedef struct rattn_args {
    const void *q;             /* [N, q_len, H_q, d] */
    const void *k_base;        /* contiguous: [H_kv, L, d]; paged: pool [n_phys_pages, H_kv, page_size, d] */
    const void *v_base;        /* same layout as k_base */
    const int32_t *block_table;/* paged: [ceil(L / page_size)] physical page of each logical page; else NULL */
    const void *lk;            /* [N, L, r], or [1, L, r] when shared_lr (NULL iff r == 0 or L == 0) */
    const void *lv;            /* same layout as lk */
    const void *bk;            /* [N, r, H_kv * d]; head k uses columns [k d, (k+1) d) (NULL iff r == 0) */
    const void *bv;            /* same layout as bk */
    const void *k_priv;        /* [N, H_kv, S, d] private keys, no residual (NULL iff S == 0) */
    const void *v_priv;        /* [N, H_kv, S, d] */
    float *out;                /* [N, q_len, H_q, d] fp32 */
    float *lse;                /* [N, q_len, H_q] fp32 natural-log sum of exp of the scores, or NULL */
    const float *v_scale;      /* RATTN_VALUES_FWHT3: [H_kv, L] fp32 scale of each value vector; else NULL */
} rattn_args;

/* Bytes of device workspace that rattn_decode (op = RATTN_OP_DECODE) or
 * rattn_prefill_chunk (op = RATTN_OP_PREFILL) needs for this descriptor.
 * Returns a rattn_status; *bytes is written on success. */
int rattn_workspace_bytes(const rattn_desc *desc, int op, size_t *bytes);

/*
 * Decode: every one of the q_len query tokens of agent a attends the L prefix
 * tokens (base + agent a's residual) and all S private tokens of agent a.
 * Two kernel launches on `stream`: split-K over the context with an online
 * softmax per split (partials in the workspace), then a merge of the splits of
 * every query row that also applies Bv once per row (LRAgent,
 * Flash-LoRA-Attention: B is applied once per query block).
 *
 * Limits (RATTN_E_UNSUPPORTED beyond them): the low-rank caches of the agents
 * that share one 16-row MFMA block group (up to 4 blocks) must span less than
 * 2 GiB (N_group * L * r * element size < 2^31).  Range (not checked): with
 * bf16 inputs each split's P V and P Lv are kept in the workspace divided by
 * the split's weight sum, as fp16, so entries of V_base, the private V and Lv
 * must lie within fp16's range (|x| <= 65504).
 *
 * Workspace: at least rattn_workspace_bytes(desc, RATTN_OP_DECODE) bytes of
 * device memory, 256-byte aligned.  Its contents on entry do not matter and are
 * scratch on exit; calls that share a workspace must not overlap in time (one
 * stream, or one workspace per stream).
 */
int rattn_decode(const rattn_desc *desc, const rattn_args *args, void *workspace, size_t workspace_bytes,
                 void *stream);

/*
 * Decode with the residual keys rebuilt per token in registers right before
 * the score product -- the ForkKV Guide's own kernel design ("Fused
 * ResidualAttention", section 2 On-the-Fly Register Fusion) -- and rotated by
 * position when rope_theta is given.  Without a rotation it computes what
 * rattn_decode computes (a variant to compare against the factored path);
 * with one it computes attention over
 *     K_a[j] = K_base[j] + rot_j(Lk_a[j] Bk_a^(k)),   V_a as in rattn_decode,
 * where rot_j rotates each pair (f, f + d/2) of a d-vector by the angle
 * j * rope_theta[f] (rotate-half rotary position embedding; K_base is taken as
 * already rotated, values are not rotated).  That is the case the factored
 * score cannot serve: (q Bk^T) Lk_j^T assumes the residual key unrotated.
 * rope_theta: NULL, or a device pointer to d/2 fp32 frequencies (radians per
 * position).  Positions are the logical prefix token indices 0 .. L-1.
 * Limits (else RATTN_E_UNSUPPORTED): bf16, head_dim 128, rank 16 or 32, a
 * contiguous base cache, priv_len 0, q_len * (H_q / H_kv) <= 16, unquantised
 * keys.  Workspace: rattn_workspace_bytes(desc, RATTN_OP_RECONSTRUCT), as in
 * rattn_decode.  Two launches (split kernel, then the decode merge).
 */
int rattn_decode_reconstruct(const rattn_desc *desc, const rattn_args *args, const float *rope_theta,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * rattn_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops or harnesses that forbid allocation): the same
 * computation and kernels, with the split partials kept in a static device
 * buffer of RATTN_NOALLOC_SCRATCH_BYTES (32 MiB) instead of a caller
 * workspace.  Each GPU the library runs on holds its own such buffer until the
 * process ends.  The call allocates and frees nothing; its first call on a
 * device looks up that device's buffer address once (hipGetSymbolAddress).
 * The buffer needs no clearing (the split launch writes every partial the
 * merge reads).  Every call on one GPU shares that GPU's buffer: calls that
 * overlap in time on one GPU (other streams, other threads) race and give
 * wrong results; order them (one stream per GPU).  Returns RATTN_E_SCRATCH,
 * launching nothing, when rattn_workspace_bytes(desc, RATTN_OP_DECODE) exceeds
 * RATTN_NOALLOC_SCRATCH_BYTES; other errors as rattn_decode.
 */
#define RATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int rattn_decode_noalloc(const rattn_desc *desc, const rattn_args *args, void *stream);

/*
 * Chunked prefill: agent a appends a chunk of C = priv_len = q_len new tokens
 * whose keys/values are k_priv/v_priv[a]; chunk query t attends the L prefix
 * tokens and chunk tokens 0..t (causal).  Same residual algebra as
 * rattn_decode (ForkKV Guide, "Mathematical Formulation of ResidualAttention";
 * LRAgent, "Flash-LoRA-Attention").  With shared_lr = 1 this is LRAgent's
 * BaseLRShared scheme ("Schemi di Condivisione"): the down-projection A is
 * shared, so one low-rank cache Lk/Lv ([1, L, r]) serves every agent's chunk
 * and only Bk/Bv differ per agent; with shared_lr = 0 it is BaseShared (one
 * low-rank cache per agent).
 * bf16 calls run one kernel that streams the whole context per block of 256
 * query rows (128 for d = 128 with r >= 64, and for d = 64 with r = 128) and
 * writes out/lse directly (no workspace:
 * rattn_workspace_bytes(desc, RATTN_OP_PREFILL) is 0, and `workspace` may be
 * NULL); fp32 calls, and paged prefixes of more than 2048 pages, run the split
 * and merge launches of rattn_decode with the causal mask (workspace as there).
 * fp32 with d = 128 and r = 128 returns RATTN_E_UNSUPPORTED (here and in
 * rattn_decode).
 */
int rattn_prefill_chunk(const rattn_desc *desc, const rattn_args *args, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * Copies the logical base cache of a paged pool into dst [H_kv, L, d] (same
 * dtype): dst[k][j] = pool[block_table[j / page_size]][k][j % page_size].
 * The block table is the list of bCache block pointers that the base-tier
 * lookup of the ForkKV Guide's DualRadixTree returns for a matched prefix
 * ("Two-Tier Lookup Mechanics", Tier 1), stored as physical page indices; the
 * pages are shared and immutable ("The Copy-on-Write Paradigm", "The
 * Disaggregated Memory Layout"), so several tables may name one page.
 * Byte-exact.  Uses desc->n_kv_heads, head_dim, prefix_len, page_size,
 * n_phys_pages, dtype.  pool, block_table and dst are device pointers (pool
 * and dst 16-byte aligned, the table 4-byte aligned); dst must not overlap
 * the pool.  Entries outside [0, n_phys_pages) are undefined behaviour.
 * prefix_len = 0 returns RATTN_OK and launches nothing; page_size must be a
 * positive multiple of 16 (else RATTN_E_UNSUPPORTED).
 */
int rattn_gather_base(const rattn_desc *desc, const void *pool, const int32_t *block_table, void *dst,
                      void *stream);

/*
 * Debug check of a block table before it is used: writes to *bad_count (a
 * device int32) the number of the ceil(prefix_len / page_size) entries of
 * block_table that lie outside [0, n_phys_pages) -- the entries whose use by
 * rattn_decode, rattn_prefill_chunk or rattn_gather_base is undefined
 * behaviour (the table holds the ForkKV Guide's bCache block pointers as
 * physical page indices, "Two-Tier Lookup Mechanics").  Reads only the table.
 * One launch on `stream`; copy the count to the host after it.  Uses
 * desc->prefix_len, page_size (a positive multiple of 16, else
 * RATTN_E_UNSUPPORTED) and n_phys_pages; prefix_len = 0 writes 0.  block_table
 * 4-byte and bad_count 4-byte aligned device pointers.
 */
int rattn_check_block_table(const rattn_desc *desc, const int32_t *block_table, int32_t *bad_count, void *stream);

/*
 * Runs selected launches of rattn_decode (op = RATTN_OP_DECODE) or
 * rattn_prefill_chunk (op = RATTN_OP_PREFILL), in their fixed order:
 *   RATTN_STAGE_SPLIT    per-split partial attention into the workspace;
 *   RATTN_STAGE_COMBINE  merge of the splits, Bv applied, out and lse written.
 * The combine reads what the split stage wrote into the same workspace (in this
 * call, or in an earlier call on the same stream with the same descriptor and
 * tensors).  stages == RATTN_STAGE_ALL is exactly rattn_decode /
 * rattn_prefill_chunk.  Lets a caller time the launches separately.  Same
 * validation and errors as the full calls; zero or bits outside
 * RATTN_STAGE_ALL return RATTN_E_SHAPE.
 */
#define RATTN_STAGE_SPLIT 1u
#define RATTN_STAGE_COMBINE 2u
#define RATTN_STAGE_ALL 3u
int rattn_attention_stages(const rattn_desc *desc, int op, const rattn_args *args, void *workspace,
                           size_t workspace_bytes, void *stream, unsigned stages);

/*
 * Base keys to int8 codes with one scale per tensor (PolyKV, section 2B: keys
 * in int8 with per-tensor linear quantisation; the shared pool is written once
 * and read by every agent).  Over the n elements at k (device, dtype
 * RATTN_BF16 or RATTN_F32, any layout: pass exactly the keys the scale must
 * cover): amax = max |k|, *scale = amax / 127 (an fp64 division rounded once to
 * fp32; 1 when amax = 0), and codes[i] = round-half-to-even(k[i] / scale) in
 * fp64, clamped to [-127, 127], stored as the byte code + 128.  scale is a
 * device pointer (one float, written on the stream; copy it to the host for
 * rattn_desc.k_scale); codes (n bytes, device) keep k's layout.  Four kernel
 * launches on `stream`; deterministic.  Inputs must be finite.
 */
int rattn_quantize_keys(const void *k, int64_t n, int32_t dtype, void *codes, float *scale, void *stream);

/*
 * Base values to 3-bit codes after a Walsh-Hadamard rotation (PolyKV, section
 * 2B, TurboQuant MSE: each value vector is rotated by a fast Walsh-Hadamard
 * transform so that its coordinates approach a standard normal, each
 * coordinate is mapped to one of eight Lloyd-Max centroids for N(0, 1), and
 * decoding looks the centroids up and undoes the rotation).  For each of the n
 * vectors v of head_dim d (64 or 128) elements at v (device, dtype RATTN_BF16
 * or RATTN_F32, vectors back to back, e.g. a [H_kv, L, d] value cache):
 *   z = H_d v, with H_d the Sylvester-ordered Hadamard matrix (entries +-1);
 *   u_j = z_j / ||v|| (0 for a zero vector), so the u_j have mean square 1;
 *   code_j = the number of inner boundaries b_1 < ... < b_7 of the 8-level
 *     minimum-MSE quantiser of N(0, 1) with u_j >= b_k (the quantiser is the
 *     fixed point of its two conditions: every centroid the N(0, 1) mean of its
 *     cell, every boundary the midpoint of its centroids; the library derives
 *     it on the host);
 *   codes (3 d / 8 bytes per vector, device): three bit planes of d / 8 bytes,
 *     plane p holding bit p of code_j at bit j % 8 of byte j / 8;
 *   scale[i] = ||v|| / d rounded once to fp32 (device, one float per vector).
 * z, ||v||, u and the comparisons are computed in fp64 (z and ||v||^2 exactly
 * for bf16 inputs).  The decoded vector is scale * H_d c, c_j the centroid of
 * code_j.  One kernel launch on `stream`; deterministic.  Inputs must be finite.
 * codes must be 8-byte aligned (rattn_decode reads them from a 16-byte aligned
 * v_base), v aligned to its element and scale to 4 bytes.
 */
int rattn_quantize_values(const void *v, int64_t n, int32_t head_dim, int32_t dtype, void *codes, float *scale,
                          void *stream);

/* The 8-level Lloyd-Max quantiser of N(0, 1) the library uses (host-only, no
 * HIP call): centroids[8] ascending and boundaries[7] ascending, in fp64. */
int rattn_values_codebook(double *centroids, double *boundaries);

/* ------------------------------------------------------------------------
 * The cache-write path: what fills the caches the attention calls read.
 * ------------------------------------------------------------------------ */

/* Shape of one low-rank projection call. */
typedef struct rattn_lr_desc {
    int32_t n_sets;    /* output sets: one low-rank cache pair per agent (BaseShared), or 1 (BaseLRShared) */
    int32_t shared_x;  /* 1: one input X for every set ([1, T, d_in]); 0: one per set */
    int32_t shared_a;  /* 1: one A for every set (Shared-A LoRA); 0: one per set */
    int32_t d_in;      /* model width the down-projection reads: a multiple of 128 */
    int32_t rank;      /* r: 8, 16, 32, 64 or 128 */
    int64_t n_tokens;  /* T >= 0 new tokens */
    int64_t pos0;      /* first cache row written (>= 0) */
    int64_t cache_len; /* rows of each set's cache: pos0 + T <= cache_len */
    int32_t dtype;     /* RATTN_BF16 (the only one supported) */
} rattn_lr_desc;

/*
 * The low-rank cache rows of T new tokens: for every set n and token t,
 *     lk[n][pos0 + t] = X_n[t] A_k,n      lv[n][pos0 + t] = X_n[t] A_v,n
 * (r values each), with X_n = x[0] when shared_x and A_.,n the set's (or the
 * shared) down-projection.  This is the LR cache of LRAgent ("Schemi di
 * Condivisione": BaseShared keeps X_i A_i per agent and recomputes it over
 * the whole context on an agent switch, the "LR prefill"; BaseLRShared
 * shares A and so one cache) and the factored residual cache X A of the
 * ForkKV Guide ("The Disaggregated Memory Layout"), which on a base hit with
 * an adapter miss is all that is computed ("Two-Tier Lookup Mechanics",
 * Case B).  The up-projections B are applied later, inside the attention.
 *
 * Layouts (device pointers, row-major, 16-byte aligned, bf16):
 *   x     [shared_x ? 1 : n_sets, T, d_in]
 *   ak_t  [shared_a ? 1 : n_sets, r, d_in]   A_k transposed (one row per rank
 *   av_t  same as ak_t                        component, as a linear layer
 *                                             d_in -> r stores its weight)
 *   lk    [n_sets, cache_len, r]   rows pos0 .. pos0 + T - 1 written, the rest untouched
 *   lv    same as lk
 * Each output value is the fp32 sum of the d_in products rounded to bf16
 * (round to nearest even).  shared_x = shared_a = 1 requires n_sets = 1.
 * One kernel launch on `stream`; T = 0 launches nothing.  Errors as the
 * attention calls (RATTN_E_UNSUPPORTED for a dtype other than bf16, d_in not a
 * multiple of 128, or another rank).
 */
int rattn_lr_project(const rattn_lr_desc *desc, const void *x, const void *ak_t, const void *av_t, void *lk,
                     void *lv, void *stream);

/*
 * Page allocator of a paged KV pool with copy-on-write (ForkKV Guide, "The
 * Copy-on-Write Paradigm"; "Reference Counting and Eviction").  A host
 * object: reference counts per physical page and a free list; it never
 * touches device memory.  Sequences that share a prefix hold the same pages
 * (retain once per sharing sequence, as a fork does); a page returns to the
 * free list when its last holder releases it.  Every call validates before
 * changing anything (a failed call changes nothing); calls on one pool may
 * come from several threads (one lock per pool).  Pages are numbered
 * 0 .. n_pages - 1 and index the pools of the attention calls.
 */
typedef struct rattn_pagepool rattn_pagepool;
int rattn_pagepool_create(int64_t n_pages, rattn_pagepool **out);
void rattn_pagepool_destroy(rattn_pagepool *pool);
/* Free pages, or a negative rattn_status. */
int64_t rattn_pagepool_free_pages(rattn_pagepool *pool);
int rattn_pagepool_refcount(rattn_pagepool *pool, int32_t page, int32_t *count);
/* n free pages, each with one reference, into pages[0 .. n-1] (RATTN_E_POOL if fewer are free). */
int rattn_pagepool_alloc(rattn_pagepool *pool, int64_t n, int32_t *pages);
/* One more reference to each listed page (each must be held); a page listed k times gains k. */
int rattn_pagepool_retain(rattn_pagepool *pool, const int32_t *pages, int64_t n);
/* One reference fewer per listing; pages reaching 0 are free again. */
int rattn_pagepool_release(rattn_pagepool *pool, const int32_t *pages, int64_t n);
/*
 * Plans the append of n_new tokens to a sequence of cur_len tokens whose
 * host block table is table[0 .. table_cap - 1]; updates the table:
 *   - the partly filled last page (cur_len % page_size != 0) is written in
 *     place when the sequence holds it alone; when it is shared, a free page
 *     becomes its private copy: *cow_src / *cow_dst name the original and the
 *     copy, the table points at the copy and the original loses this
 *     sequence's reference (else both are -1);
 *   - every further page the new tokens reach comes from the free list.
 * The caller then copies the table to the device and runs rattn_append_kv
 * with the same cur_len, n_new and cow pages.  RATTN_E_POOL (nothing changed)
 * when the free pages do not suffice; RATTN_E_SHAPE when the table is too
 * short or names a page the pool does not hold.
 */
int rattn_pagepool_plan_append(rattn_pagepool *pool, int32_t *table, int64_t table_cap, int64_t cur_len,
                               int64_t n_new, int32_t page_size, int32_t *cow_src, int32_t *cow_dst);

/*
 * The data movement of a planned append, on the device: writes the T = n_new
 * new rows of every KV head, k_new/v_new [H_kv, T, d] (device, same dtype as
 * the pools), at logical positions cur_len .. cur_len + T - 1 of the sequence
 * whose updated block table is `table` (device, int32, >= ceil((cur_len + T)
 * / page_size) entries), into both pools [n_phys_pages, H_kv, page_size, d];
 * and, when cow_src >= 0, first fills rows 0 .. (cur_len % page_size) - 1 of
 * every head of page cow_dst from page cow_src (the private copy keeps the
 * rows the original held).  Uses desc->n_kv_heads, head_dim, page_size,
 * n_phys_pages and dtype.  One kernel launch; byte-exact.  The table's
 * entries and the cow pages must lie in [0, n_phys_pages) (cow pages checked
 * on the host, table entries not).  k_new/v_new must not overlap the pools.
 */
int rattn_append_kv(const rattn_desc *desc, void *pool_k, void *pool_v, const int32_t *table, int64_t cur_len,
                    int64_t n_new, const void *k_new, const void *v_new, int32_t cow_src, int32_t cow_dst,
                    void *stream);

/* Work decomposition chosen for a call (host-only introspection; no HIP call).
 * The kernel that runs is determined by (dtype, head_dim, path, resid_cols,
 * masked, waves): path 0 is the split kernel (waves > 8 selects its twelve-wave
 * form) followed by the merge; path 1 is the prefill kernel. */
typedef struct rattn_plan_info {
    int32_t n_prefix_splits;  /* context splits of the prefix */
    int64_t prefix_split_len; /* tokens per prefix split */
    int32_t n_priv_splits;    /* splits of each agent's private tokens */
    int64_t priv_split_len;
    int32_t row_blocks;       /* 16-row MFMA blocks per KV head over the prefix */
    int32_t agents_per_block; /* agents whose query rows share one block */
    int32_t resid_cols;       /* residual columns per block, padded (0 if r == 0) */
    int32_t work_items;       /* workgroups of the split (or prefill) kernel */
    int32_t heads_per_item;   /* KV heads one prefix workgroup serves (sharing its low-rank tile) */
    int32_t waves;            /* waves per workgroup (compute + load) */
    int32_t masked;           /* 1: per-agent caches, several agents per block, residual columns = rank */
    int32_t blocks_per_group; /* row blocks one prefix workgroup serves */
    int32_t path;             /* 0: split kernel + merge; 1: prefill kernel (no workspace) */
    int32_t rows_per_item;    /* path 1: query rows of one (KV head, agent) per workgroup; else 0 */
} rattn_plan_info;

/* The plan of rattn_decode (rattn_decode_plan) or of rattn_prefill_chunk
 * (rattn_prefill_plan) for this descriptor.  Same validation as the calls;
 * a rattn_status is returned and *info written on success. */
int rattn_decode_plan(const rattn_desc *desc, rattn_plan_info *info);
int rattn_prefill_plan(const rattn_desc *desc, rattn_plan_info *info);

const char *rattn_status_str(int status);
int rattn_version(void);
/* hipError_t of the calling thread's last RATTN_E_HIP, or 0. */
int rattn_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RATTN_H */
