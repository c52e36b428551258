/*
 * fd.h -- split-KV single-query decode attention (Flash-Decoding) for
 * AMD Instinct MI355X (gfx950).  C ABI of libfd.so.
 *
 * The operation.  "Flash-Decoding for long-context inference" (Dao,
 * Haziza, Massa, Sizov; Stanford CRFM blog), section "Multi-head attention
 * for decoding": at each decoding step the single new query of every head
 * attends to all tokens already in the KV cache.  For every batch entry b
 * and query head h, with kv-head g = h / (Hq / Hkv) and L = seqlens[b]:
 *
 *     s_j      = scale * <q[b,h,:], k_cache[b,g,j,:]>      0 <= j < L
 *     out[b,h] = sum_j softmax(s)_j * v_cache[b,g,j,:]
 *     lse[b,h] = ln sum_j exp(s_j)                         (natural log)
 *     L == 0  ->  out = 0, lse = -inf
 *
 * No mask beyond the valid length: the current token's K/V is expected to
 * be in the cache already.
 *
 * How it is computed.  Same page, section "A faster attention for
 * decoding: Flash-Decoding": the keys/values of each sequence are cut into
 * chunks that are processed in parallel, each writing its partial output
 * and one log-sum-exp per query row; a small final reduction rescales the
 * chunks by their log-sum-exp and sums them.  The number of chunks is
 * chosen for the GPU's compute-unit count so that even batch 1 fills the
 * chip.  When one chunk per sequence already fills it, the partials are
 * skipped and the single pass writes out/lse directly (the pages' choice
 * between Flash-Decoding and plain FlashAttention by problem size).  The
 * final reduction is a second, small kernel on the same stream; with
 * FD_FLAG_FUSED_MERGE it runs inside the first launch instead, by the last
 * workgroup to finish each (sequence, KV head) group.
 *
 * Layouts (all contiguous, row-major, element type `dtype` unless noted):
 *     q        [B][Hq][D]
 *     k_cache  [B][Hkv][Lmax][D]     head-major: each (b, g) is one slab
 *     v_cache  [B][Hkv][Lmax][D]
 *     seqlens  int32 [B], DEVICE memory, or NULL (= every sequence is Lmax)
 *     out      [B][Hq][D]
 *     lse      float32 [B][Hq]
 * Rows j >= seqlens[b] of a slab are never read (they may hold anything,
 * NaN included).  Pointers must be 16-byte aligned device pointers.
 *
 * Supported: D in {64, 128, 256} (256: the matrix-core kernels only);
 * dtype FD_BF16, FD_F16 or FD_F32; 1 <= Hq/Hkv <= 128;
 * Lmax <= 2^30 keys.  A KV head serves up to 16 query rows per workgroup
 * (the matrix cores' q-tile); a larger group runs as the fewest equal
 * groups that fit, each reading the KV head's rows again (so K/V bytes are
 * read that many times).  bf16 and fp16 scores and outputs are accumulated
 * in fp32; a 16-bit output is rounded to nearest even.
 *
 * Ownership.  The caller owns every buffer.  `stream` is a hipStream_t
 * passed as void* (NULL = the default stream).  The library keeps no
 * pointer to a caller's buffer after a call returns; the only memory it
 * holds is its own workspace (calls given no workspace use it).  Calls plan for the current HIP
 * device (its compute-unit count) and keep that workspace on it, so the
 * current device must be the one that holds the buffers and the stream.
 * out and lse must not overlap each other, an input or the workspace (the
 * kernels read the inputs while they write the outputs); inputs may share
 * memory, since they are only read.
 *
 * Errors.  Every entry point returns FD_OK or a negative FD_ERR_* code;
 * argument checks run on the host before anything is launched, and nothing
 * is launched when one fails.  No C++ exception crosses the ABI.
 *
 * Synchronisation.  Calls are asynchronous on `stream`; results are valid
 * once the stream's work has completed.  The library does not synchronise
 * (the one exception: when its own workspace grows, freeing the old buffer
 * waits for the device), so it cannot validate the device-side seqlens: a
 * value outside [0, Lmax] is a caller error that the kernels clamp into
 * that range.
 *
 * Graph capture.  A call with a caller workspace (or whose plan needs no
 * workspace) queues kernels only and may be captured in a HIP graph.  A
 * call that would use the library-owned workspace returns FD_ERR_CAPTURE
 * while `stream` is capturing: a later call may free and replace that
 * buffer, which a graph must not hold.
 *
 * Symbols.  libfd.so exports exactly the functions declared here.
 */
#ifndef FD_H
#define FD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Marks the exported entry points (the library is built with every other
   symbol hidden). */
#ifndef FD_API
#define FD_API __attribute__((visibility("default")))
#endif

typedef enum fd_dtype {
    FD_BF16 = 0, /* bfloat16 q/k/v/out */
    FD_F32 = 1,  /* float32 q/k/v/out */
    FD_F16 = 2   /* IEEE binary16 q/k/v/out */
} fd_dtype_t;

enum {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = -1, /* NULL pointer, non-positive size, Hq % Hkv,
                                non-finite scale, misaligned pointer */
    FD_ERR_UNSUPPORTED = -2, /* D, dtype, group size or Lmax outside the
                                supported range */
    FD_ERR_WORKSPACE = -3,   /* caller workspace too small / alloc failed */
    FD_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
    FD_ERR_CAPTURE = -5,     /* the library-owned workspace was needed while
                                `stream` is capturing a graph */
    FD_ERR_TOO_LARGE = -6    /* fd_decode_noalloc: the plan's partials do
                                not fit FD_NOALLOC_SCRATCH_BYTES */
};

/* Flags of fd_decode_ex / fd_plan. */
enum {
    /* Merge the chunks inside the per-chunk launch: the last workgroup of
       each (b, KV head) group, found with a ticket counter, merges it.
       The partials then cross MI355X's eight L2 caches as write-through
       stores, and one workgroup per group merges them at the end of the
       launch; measured slower than the separate merge kernel at batch 1,
       so the planner never picks it by itself.  For callers that must
       have a single launch. */
    FD_FLAG_FUSED_MERGE = 1,
    /* Always leave per-chunk partials, even when one chunk per sequence
       would do (the plan fd_decode_partials / fd_merge_partials use). */
    FD_FLAG_PARTIALS = 2,
    /* Unified-maximum softmax (fd_decode_unified_max sets it; fd_plan and
       fd_plan_ex accept it; other calls reject it). */
    FD_FLAG_UNIFIED_MAX = 4
};

/* How the chunks of a split plan are merged (fd_plan_t.merge). */
enum {
    FD_MERGE_NONE = 0,     /* one chunk per sequence: no partials */
    FD_MERGE_FUSED = 1,    /* last workgroup of each group merges */
    FD_MERGE_SEPARATE = 2  /* a second kernel merges */
};

/* Kernel variant chosen for the per-chunk pass. */
enum {
    FD_VARIANT_AUTO = 0,
    FD_VARIANT_MFMA = 1, /* matrix-core pass, q group padded to 16 (any
                            dtype; paged and several tokens: always) */
    FD_VARIANT_VALU = 2  /* vector-ALU pass (fp32, or 16-bit small groups) */
};

/* What the planner decided for one problem shape (filled by fd_plan). */
typedef struct fd_plan_info {
    int num_splits;      /* chunks per sequence of length Lmax (S) */
    int chunk;           /* keys per chunk (C), a multiple of 32 */
    int variant;         /* FD_VARIANT_MFMA or FD_VARIANT_VALU */
    int waves_per_block; /* 64-lane wavefronts per workgroup */
    int grid;            /* workgroups of the per-chunk pass; with seqlens
                            the chunk count is an upper bound, and the
                            matrix-core pass launches max(half of it, 8
                            per CU), workgroup i taking chunks i and
                            i + grid */
    int combine;         /* 1 if chunks leave partials to be merged */
    int merge;           /* FD_MERGE_NONE / _FUSED / _SEPARATE */
    int num_cus;         /* compute units the plan was sized for */
    size_t workspace_bytes; /* tickets + partials the plan needs */
    size_t ticket_bytes;    /* leading bytes of the workspace that hold the
                               per-group tickets of the fused merge
                               (0 unless FD_FLAG_FUSED_MERGE) */
    size_t o_part_offset;   /* byte offset of the partial outputs, each
                               chunk's own softmax-normalised output,
                               float32, laid out as partial_layout says */
    size_t lse_part_offset; /* byte offset of the partial log-sum-exps,
                               float32, natural log, same layout without
                               the D axis; chunk s of sequence b exists iff
                               s < max(1, ceil(seqlens[b] / chunk)) */
    int partial_layout;     /* FD_PARTIALS_ROW_MAJOR or _CHUNK_MAJOR */
    int partial_group;      /* P: query heads per group of the chunk-major
                               layout: G = Hq / Hkv, or G / r when a KV
                               head's G * Tq query rows run as r groups
                               (more than 16 rows on the matrix cores;
                               groups past 8 heads on the vector ALU) */
} fd_plan_t;

/* Layouts of the chunk partials (fd_plan_t.partial_layout), with S =
   num_splits, P = fd_plan_t.partial_group, Tq query tokens per sequence
   (1 for decode):
     FD_PARTIALS_ROW_MAJOR    o_part [B][Tq][Hq][S][D], lse_part
                              [B][Tq][Hq][S]: a query row's chunks together
                              (plans whose chunks all run in one round of
                              workgroups);
     FD_PARTIALS_CHUNK_MAJOR  o_part [B][Hq/P][S][Tq][P][D], lse_part
                              [B][Hq/P][S][Tq][P]: one chunk's rows of a
                              group of P query heads together (plans that
                              run in several rounds); P = Hq / Hkv unless a
                              KV head's rows are split (see partial_group). */
enum {
    FD_PARTIALS_ROW_MAJOR = 0,
    FD_PARTIALS_CHUNK_MAJOR = 1
};

/*
 * fd_decode -- out, lse = attention(q, k_cache, v_cache) as defined above.
 * Uses a workspace owned by the library: allocated on first use per
 * device and grown when a larger problem needs it (that call allocates
 * and synchronises; the others queue kernels only).  Calls on different
 * streams of one device must not overlap, since they share that
 * workspace.  Under stream capture: FD_ERR_CAPTURE whenever the plan needs
 * a workspace (see "Graph capture").  Results do not depend on the order
 * in which workgroups finish: for a given plan the output is bitwise
 * reproducible.
 */
FD_API int fd_decode(const void *q, const void *k_cache,
                     const void *v_cache, const int32_t *seqlens, int B,
                     int Hq, int Hkv, int D, int Lmax, float scale,
                     fd_dtype_t dtype, void *out, float *lse, void *stream);

/*
 * fd_decode_ex -- as fd_decode, with the caller's choices:
 *   num_splits  0 = planner's choice, else chunks per Lmax-long sequence
 *               (clamped to [1, ceil(Lmax / 32)]); 1 disables the merge.
 *   variant     FD_VARIANT_AUTO / _MFMA / _VALU.  AUTO: the matrix cores
 *               for bf16 and fp16, and for fp32 from groups of 3 query
 *               heads (at D = 64 also smaller groups from Lmax = 4096);
 *               the vector ALU for the other fp32 shapes.  VALU takes
 *               16-bit groups of at most 4 heads only.
 *   flags       0 or FD_FLAG_FUSED_MERGE.
 *   workspace   device buffer of at least fd_workspace_bytes(...) bytes
 *               for the same arguments, 256-byte aligned, or NULL with
 *               workspace_bytes 0 to use the library-owned one.  A caller
 *               workspace makes the call allocation-free and free of
 *               library state, so it can be captured in a HIP graph and
 *               replayed (it queues kernels only; no memset, no copy).
 *               With FD_FLAG_FUSED_MERGE its first
 *               fd_plan_t.ticket_bytes bytes are per-group tickets that must
 *               be zero when a call starts: zero-fill a new workspace once;
 *               every call leaves its tickets zero again, but the rest of
 *               the buffer holds partials, so zero-fill again before reusing
 *               it for a fused call with a larger B * Hkv.
 */
FD_API int fd_decode_ex(const void *q, const void *k_cache,
                        const void *v_cache, const int32_t *seqlens, int B,
                        int Hq, int Hkv, int D, int Lmax, float scale,
                        fd_dtype_t dtype, void *out, float *lse,
                        int num_splits, int variant, int flags,
                        void *workspace, size_t workspace_bytes,
                        void *stream);

/* Size of fd_decode_noalloc's fixed scratch array, per device. */
#define FD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * fd_decode_noalloc -- fd_decode_ex for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no hipMalloc, hipFree or allocating
 * library routine and takes no workspace: the chunk partials live in a
 * fixed device array inside the library, FD_NOALLOC_SCRATCH_BYTES (64 MiB)
 * on each device, held until the process ends.  A plan whose partials
 * need more (fd_plan(...).workspace_bytes > FD_NOALLOC_SCRATCH_BYTES)
 * returns FD_ERR_TOO_LARGE before anything is launched; a single-pass
 * plan needs none.  The first call on a device looks up that device's
 * copy of the array (no allocation, no work queued).
 *   num_splits, variant  as for fd_decode_ex
 *   flags                0 or FD_FLAG_PARTIALS; FD_FLAG_FUSED_MERGE is
 *                        FD_ERR_UNSUPPORTED (its tickets would have to be
 *                        zeroed by every call), FD_FLAG_UNIFIED_MAX
 *                        FD_ERR_INVALID_ARG
 * Every call on one device shares that device's array, which keeps the
 * last call's partials; nothing in it needs to start at zero.  Calls that
 * overlap on one device (different streams without ordering between them)
 * race on it and give undefined results: serialise them.  Queues kernels
 * only, so it can be captured in a HIP graph; a replay uses the array as
 * any other call on that device does.
 */
FD_API int fd_decode_noalloc(const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *seqlens,
                             int B, int Hq, int Hkv, int D, int Lmax,
                             float scale, fd_dtype_t dtype, void *out,
                             float *lse, int num_splits, int variant,
                             int flags, void *stream);

/*
 * fd_decode_partials / fd_merge_partials -- the two phases of a split decode
 * as separate calls: the parallel pass over the chunks, and the log-sum-exp
 * reduction (the two steps of the Flash-Decoding section), for callers that
 * schedule or time them apart, or merge partials gathered elsewhere.
 * Both plan with FD_FLAG_PARTIALS added to `flags`, so partials exist even
 * for one chunk per sequence; use fd_plan / fd_workspace_bytes with that
 * flag for the layout and size of `workspace` (a caller buffer, required).
 * fd_merge_partials must get the same sizes, seqlens, num_splits, variant
 * and flags as the fd_decode_partials call that filled the workspace, and
 * run after it (same stream, or ordered by the caller).
 */
FD_API int fd_decode_partials(const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *seqlens,
                              int B, int Hq, int Hkv, int D, int Lmax,
                              float scale, fd_dtype_t dtype, int num_splits,
                              int variant, int flags, void *workspace,
                              size_t workspace_bytes, void *stream);

FD_API int fd_merge_partials(const int32_t *seqlens, int B, int Hq, int Hkv,
                             int D, int Lmax, fd_dtype_t dtype,
                             int num_splits, int variant, int flags,
                             const void *workspace, size_t workspace_bytes,
                             void *out, float *lse, void *stream);

/*
 * fd_plan -- the decision fd_decode_ex would take, without launching.
 * varlen: nonzero when seqlens will be passed (chunks are then sized for
 * a mix of lengths).  num_cus: compute units to plan for; 0 queries the
 * current HIP device.  Returns FD_OK or an FD_ERR_* code (plan untouched).
 */
FD_API int fd_plan(int B, int Hq, int Hkv, int D, int Lmax, fd_dtype_t dtype,
                   int varlen, int num_splits, int variant, int flags,
                   int num_cus, fd_plan_t *plan);

/* Page-pool layouts of fd_decode_paged. */
enum {
    FD_PAGES_TOKEN_MAJOR = 0, /* [num_pages][page_size][Hkv][D] */
    FD_PAGES_HEAD_MAJOR = 1   /* [num_pages][Hkv][page_size][D] */
};

/*
 * fd_decode_paged -- the same attention over a paged KV cache.  The
 * "flash decoding" search-result page (a note on decode kernels for
 * serving) observes that frameworks store the KV cache in very different
 * ways; vLLM-style paging is the common one: fixed-size pages in a shared
 * pool and a per-sequence table of page indices.
 *     k_pages, v_pages  pools of num_pages pages (dtype), `layout`:
 *         FD_PAGES_TOKEN_MAJOR  [num_pages][page_size][Hkv][D]
 *         FD_PAGES_HEAD_MAJOR   [num_pages][Hkv][page_size][D]
 *     block_table       int32 [B][max_pages], DEVICE memory
 *     seqlens           int32 [B], DEVICE memory, REQUIRED
 *     q, out, lse       as for fd_decode when Tq = 1; for Tq > 1 causal new
 *                       tokens per sequence as for fd_decode_multiquery:
 *                       q, out [B][Tq][Hq][D], lse [B][Tq][Hq]
 * Token j < L = clamp(seqlens[b], 0, max_pages * page_size) of sequence b,
 * KV head g, is in page pg = block_table[b][j / page_size] at t = j %
 * page_size: row ((pg * page_size + t) * Hkv + g) * D token-major,
 * ((pg * Hkv + g) * page_size + t) * D head-major; the result is
 * fd_decode's over those rows.  Head-major pages keep each head's rows of
 * a page together and stream faster on MI355X.  Only the first
 * ceil(L / page_size) table entries of a sequence are read, and only rows
 * below L of its last page.  page_size must be a multiple of 16
 * (FD_ERR_UNSUPPORTED otherwise), max_pages * page_size and num_pages *
 * page_size * Hkv at most INT_MAX.  A table entry outside [0, num_pages)
 * is a caller error that the kernel clamps into that range (never a read
 * outside the pools).
 * FD_BF16, FD_F16 or FD_F32 (all on the matrix cores), 1 <= Tq <= 16;
 * groups of more than 16 query rows (Tq * Hq/Hkv) are split as for
 * fd_decode.
 * num_splits, flags: as for fd_decode_ex (chunks per max_pages * page_size
 * tokens; FD_FLAG_FUSED_MERGE allowed).  workspace, workspace_bytes: as
 * for fd_decode_ex, sized by fd_plan_ex(B, Tq, Hq, Hkv, D,
 * max_pages * page_size, dtype, 1, 1, num_splits, FD_VARIANT_AUTO, flags,
 * 0, &plan).workspace_bytes; NULL and 0 use the library-owned one.
 */
FD_API int fd_decode_paged(const void *q, const void *k_pages,
                           const void *v_pages, const int32_t *block_table,
                           int max_pages, int page_size, int num_pages,
                           int layout, const int32_t *seqlens, int B, int Tq,
                           int Hq, int Hkv, int D, float scale,
                           fd_dtype_t dtype, void *out, float *lse,
                           int num_splits, int flags, void *workspace,
                           size_t workspace_bytes, void *stream);

/*
 * fd_decode_multiquery -- Tq new query tokens per sequence at once (the
 * same search-result note: multi-turn chat and speculative decoding give
 * several query vectors per step, which raises the work per byte read).
 * The Tq tokens are the newest of each sequence and their K/V are already
 * the last Tq rows of the cache; attention among them is causal:
 *     q, out   [B][Tq][Hq][D]      lse  float32 [B][Tq][Hq]
 *     k_cache, v_cache, seqlens    as for fd_decode
 * Query token t < Tq of sequence b sees keys j < L - (Tq - 1 - t), with
 * L = clamp(seqlens[b], 0, Lmax) (NULL seqlens: L = Lmax); a token that
 * sees no key gets out = 0, lse = -inf.  Tq = 1 is fd_decode.
 * The keys a token must not see (j in [L - Tq + 1, L)) are still loaded
 * for the tile and weighted by exactly 0: their V rows must be finite.
 * FD_BF16, FD_F16 or FD_F32, 1 <= Tq <= 16.  The Tq * Hq/Hkv query rows of
 * a KV head share one 16-column matrix-core tile, or, when there are more, the
 * fewest equal groups of them that fit (each reading the KV head's rows);
 * with Tq = 1 fp32 may run on the vector ALU, as in fd_decode.  num_splits, flags and the workspace
 * as for fd_decode_ex, sized by fd_plan_ex(B, Tq, Hq, Hkv, D, Lmax, dtype,
 * seqlens != NULL, 0, num_splits, FD_VARIANT_AUTO, flags, 0,
 * &plan).workspace_bytes.
 */
FD_API int fd_decode_multiquery(const void *q, const void *k_cache,
                                const void *v_cache, const int32_t *seqlens,
                                int B, int Tq, int Hq, int Hkv, int D,
                                int Lmax, float scale, fd_dtype_t dtype,
                                void *out, float *lse, int num_splits,
                                int flags, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * fd_decode_unified_max -- fd_decode_ex computed with FlashDecoding++'s
 * asynchronised softmax ("FlashDecoding++: Faster Large Language Model
 * Inference on GPUs", summarised on the "flash decoding" search-result
 * page, which names the cost it removes: partial softmax results that
 * must be synchronised with each other).  Each chunk takes its
 * exponentials against one fixed estimate phi of the row maximum instead
 * of a running maximum, so tiles need no cross-lane maximum and no
 * rescaling of their sums.  phi is in the units of lse (natural log of
 * the scaled score), chosen by the caller from the model's score range
 * (0 suits unit-variance scores).  Fallback: when the largest score of
 * some row of a chunk lies outside phi +- 64 ln 2 (bf16) or outside
 * [phi, phi + 14 ln 2] (fp16), where 2^x would overflow or lose
 * precision, that
 * chunk is recomputed with the running maximum, giving exactly the
 * fd_decode_ex result for it; either way the result is the same
 * attention within the usual rounding.  Contiguous cache, one token per
 * sequence, bf16 or fp16 only (FD_ERR_UNSUPPORTED otherwise).  phi must be
 * finite.
 * num_splits, flags (FD_FLAG_FUSED_MERGE), workspace: as for
 * fd_decode_ex; plan with FD_FLAG_UNIFIED_MAX for the workspace size.
 */
FD_API int fd_decode_unified_max(const void *q, const void *k_cache,
                                 const void *v_cache, const int32_t *seqlens,
                                 int B, int Hq, int Hkv, int D, int Lmax,
                                 float scale, fd_dtype_t dtype, void *out,
                                 float *lse, float phi, int num_splits,
                                 int flags, void *workspace,
                                 size_t workspace_bytes, void *stream);

/*
 * fd_plan_ex -- fd_plan for the calls above: Tq query tokens per sequence
 * (1 for fd_decode), paged nonzero for a paged cache
 * (then Lmax = max_pages * page_size and seqlens are implied).  The
 * partial layouts carry the token index as fd_plan_t.partial_layout shows.
 */
FD_API int fd_plan_ex(int B, int Tq, int Hq, int Hkv, int D, int Lmax,
                      fd_dtype_t dtype, int varlen, int paged, int num_splits,
                      int variant, int flags, int num_cus, fd_plan_t *plan);

/*
 * fd_workspace_bytes -- bytes of device workspace fd_decode_ex needs for
 * these arguments on the current device (0 when no merge pass is needed).
 * Returns 0 as well for invalid arguments; fd_plan reports why.
 */
FD_API size_t fd_workspace_bytes(int B, int Hq, int Hkv, int D, int Lmax,
                                 fd_dtype_t dtype, int varlen, int num_splits,
                                 int variant, int flags);

/* Static English text for a status code. */
FD_API const char *fd_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
FD_API int fd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H */
