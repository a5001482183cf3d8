/*
 * zha.h -- C ABI of the Zyphra Hierarchical Attention (ZHA) decode path on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (page references are by site and section heading):
 *   [wqu]   wqu.guru, "Zyphra发布层级注意力ZHA：稀疏搜索实现亚二次复杂度"
 *   [flux]  fluxbbs.com, "Zyphra ZHA 稀疏注意力：8.2 万参数与 373 倍加速推算"
 *   [aitop] aitop.news, "Zyphra 提出树结构索引器 ZHA，实现亚二次复杂度长上下文注意力"
 *           (the paper's abstract)
 *   [icwork] ic.work article on ZHA
 * Keys of one attention layer's KV cache are cut into chunks of C tokens;
 * every chunk, and recursively every group of C nodes, is summarised by R
 * tangent planes of its log attention mass, one per reference query
 * ([wqu] "Building the tree").  A decode query scores the top nodes, keeps the
 * smallest set holding a fraction p of the estimated mass, expands only those
 * nodes' children and repeats down to raw chunks ([wqu] "How does top-p routing
 * pick tokens?"); exact attention then reads only the kept chunks plus the
 * first token ([wqu] same section; "What is Zyphra Hierarchical Attention").
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers unless a comment says "host".  All
 *     device work is enqueued on the given stream; no entry point synchronises
 *     the host with the device, allocates device memory after
 *     zha_tree_create, or issues memset nodes, so a call sequence can be
 *     captured into a HIP graph.
 *   - B sequences, Hkv KV heads, Hq = G * Hkv query heads (query head h reads
 *     KV head h / G), head dimension d.  A "unit" is one (sequence, KV head).
 *   - K and V: [B][Hkv][max_tokens][d], contiguous, dtype of the tree.  q:
 *     [B][Hq][d], same dtype.  refs: [Hkv][R][d] float32.  out: [B][Hq][d]
 *     float32.  lse: [B][Hq] float32.  All owned by the caller.
 *   - Logits are scale * q.k; the tree's planes live in scaled-query space, so
 *     zha_route and zha_attend must receive the same scale.
 *   - Level 1 nodes are leaf chunks of C consecutive tokens; a level-l node
 *     covers C^l tokens; only complete leaf chunks enter the tree (the tree
 *     spans Nc = C*floor(N/C) tokens; the last node of a level may be partial).
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a failed validation returns a status and enqueues nothing.
 *     A failed launch returns ZHA_ERR_HIP.  Faults inside kernels surface at
 *     the caller's next synchronisation of the stream.  No exception crosses
 *     the ABI.  A tree is not thread-safe; distinct trees are independent.
 */
#ifndef ZHA_H
#define ZHA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point below is exported from libzha.so with default visibility. */
#define ZHA_API __attribute__((visibility("default")))

typedef struct zha_tree* zha_tree_t;

typedef enum {
    ZHA_OK = 0,
    ZHA_ERR_INVALID = 1,      /* an argument is out of range or null */
    ZHA_ERR_CAPACITY = 2,     /* a length exceeds the tree's max_tokens */
    ZHA_ERR_NOMEM = 3,        /* device or host allocation failed */
    ZHA_ERR_UNSUPPORTED = 4,  /* a shape the library does not implement */
    ZHA_ERR_HIP = 5,          /* a HIP runtime call failed */
    ZHA_ERR_DEVICE = 6        /* a device-side bounded wait gave up (see zha_tree_check) */
} zha_status;

typedef enum { ZHA_F32 = 0, ZHA_BF16 = 1 } zha_dtype;

/* Storage of the planes' m.  ZHA_SUMMARY_NATIVE: m in the tree dtype.
 * ZHA_SUMMARY_FP8 (tree dtype bf16 only): a low-precision router summary
 * ([wqu] opening bullets: a router variant in a 4-bit format was also tested;
 * the pages give no format; the library offers 8 bits here and 4 bits below).  Each (node, reference)
 * row of d values is stored as OCP fp8 e4m3 codes times a power-of-two scale
 * 2^e, e the smallest integer with max|m| * 2^-e <= 448; each value m * 2^-e is
 * rounded to the nearest e4m3 value (ties to even mantissa, subnormals kept).
 * b = LSE - r.m~ is formed from the decoded m~ = code * 2^e, as for native
 * storage, so every plane stays exact at q = r.  A level-1 node then takes
 * R * (d + 8) bytes instead of R * (2d + 4).
 * ZHA_SUMMARY_FP4 (tree dtype bf16 only): the 4-bit reading.  Each row is cut
 * into blocks of 32 consecutive values, each stored as OCP fp4 e2m1 codes
 * (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; two per byte, element 2i in the low
 * nibble of byte i) times its own power-of-two scale 2^e, e the smallest
 * integer with max|m_block| * 2^-e <= 6 (kept as the byte e + 127); values
 * rounded to the nearest e2m1 value, ties to even mantissa.  b is formed from
 * the decoded m~ as above.  A level-1 node takes R * (d/2 + d/32 + 4) bytes. */
typedef enum { ZHA_SUMMARY_NATIVE = 0, ZHA_SUMMARY_FP8 = 1, ZHA_SUMMARY_FP4 = 2 } zha_summary;

/* Shape of one layer's tree.  Supported: head_dim in {64, 128};
 * n_refs in {1, 2, 4, 8, 16}; group = n_q_heads / n_kv_heads in [1, 16];
 * chunk >= 2; 1 <= levels <= 16 with chunk^levels <= 2^30; max_tokens < 2^31. */
typedef struct {
    int32_t batch;        /* B */
    int32_t n_kv_heads;   /* Hkv */
    int32_t n_q_heads;    /* Hq, a multiple of Hkv */
    int32_t head_dim;     /* d */
    int32_t chunk;        /* C: tokens per leaf chunk and children per node */
    int32_t levels;       /* L: summary levels */
    int32_t n_refs;       /* R: reference queries per KV head */
    int64_t max_tokens;   /* capacity per sequence (the K/V token stride) */
    zha_dtype dtype;      /* storage dtype of q, K and V, and of the planes' m when native */
    zha_summary summary;  /* storage of the planes' m (fp8 and fp4 need dtype bf16) */
    int32_t per_head_routes; /* nonzero: the tree also serves ZHA_ROUTE_PER_HEAD routes (its
                                routing workspace is sized for B*Hq routing units) */
    int32_t max_queries;  /* queries per sequence one zha_route_multi may carry (0 is taken
                             as 1); the routing workspace is sized for that many.  The routing
                             units of the largest route must number at most 65535 */
} zha_tree_desc;

/* How the G query heads of one KV head are routed.  ZHA_ROUTE_GROUP: one kept
 * set per (sequence, KV head), from the mean over the G heads of each head's
 * frontier-normalised mass (the reading taken for grouped-query attention).
 * ZHA_ROUTE_PER_HEAD: every query head is routed alone, as the pages describe
 * routing for a single query ([wqu] "How does top-p routing pick tokens?"): one
 * kept set per (sequence, query head), and attention of each head over its own
 * set.  A "routing unit" is a (sequence, KV head) in group mode and a
 * (sequence, query head) in per-head mode, numbered (b, KV head, head in group)
 * with the head fastest (zha_route_multi adds the query of the block, see
 * there).  Routing units that share one KV head's planes may be scored
 * together (one load of each plane for all of them) and attended together
 * (one load of each K/V row); every unit's kept set and output are those it
 * would get alone. */
typedef enum { ZHA_ROUTE_GROUP = 0, ZHA_ROUTE_PER_HEAD = 1 } zha_route_mode;

/* Kept leaf chunks of the last route on a tree: a view into the tree's
 * workspace, valid until the next route on the same tree.
 * counts: device [routing units]; ids: device [routing units][cap], each
 * unit's ids ascending ([B*Hkv] for zha_route). */
typedef struct {
    const int32_t* counts;
    const int32_t* ids;
    int64_t cap;
} zha_kept;

/* Allocates a tree and all its device workspace for the descriptor (the
 * planes of every level, the fp32 accumulators of each unit's rightmost open
 * nodes, and the routing/attention scratch).  The current HIP device owns it.
 * Errors: ZHA_ERR_INVALID (null or out-of-range field), ZHA_ERR_UNSUPPORTED,
 * ZHA_ERR_NOMEM. */
ZHA_API zha_status zha_tree_create(const zha_tree_desc* desc, zha_tree_t* out);
ZHA_API void zha_tree_destroy(zha_tree_t tree);

/* Device bytes held by the tree (planes + accumulators + workspace). */
ZHA_API zha_status zha_tree_bytes(zha_tree_t tree, int64_t* bytes);

/* Builds every level's planes from the caller's keys ([wqu] "Building the
 * tree"; [aitop] abstract: recursively compressed key summaries).  For each
 * node and reference query r the node stores m_r (the r-softmax-weighted mean
 * key, in the tree dtype) and b_r = LSE_r - r.m_r (float32, from the stored
 * m_r), LSE_r being the log-sum-exp of r.k over the node's tokens.  Parents
 * combine their children's fp32 (LSE, mean) exactly; leaves read K once.
 * refs are copied into the tree.  seq_lens (host [B]) sets each sequence's
 * length N_b, 1 <= N_b <= max_tokens.
 * Errors: ZHA_ERR_INVALID, ZHA_ERR_CAPACITY, ZHA_ERR_HIP. */
ZHA_API zha_status zha_build(zha_tree_t tree, const void* K, const float* refs,
                     const int32_t* seq_lens, hipStream_t stream);

/* Grows the tree after the caller has written rows [N_b, new_N_b) of K (and
 * V).  Every leaf chunk completed by the new rows gets its planes, is folded
 * into its ancestors' fp32 accumulators in order, and the planes of the
 * affected ancestors (complete or still open) are rewritten.  The result is
 * bit-identical to zha_build over the grown cache.  new_seq_lens: host [B],
 * N_b <= new_N_b <= max_tokens.  The tree reading of growth is not stated on
 * the pages, which only say that future queries traverse a tree built over
 * the KV cache ([aitop] abstract).
 * Errors: ZHA_ERR_INVALID (shrinking length or no prior zha_build),
 * ZHA_ERR_CAPACITY, ZHA_ERR_HIP. */
ZHA_API zha_status zha_append(zha_tree_t tree, const void* K, const int32_t* new_seq_lens,
                      hipStream_t stream);

/* Routes the Hq decode queries top-down ([wqu] "How does top-p routing pick
 * tokens?").  For each unit and level, every frontier node i is scored for
 * each of the G query heads of the KV head as s_hi = max_r (b_ir + scale *
 * q_h.m_ir); each head's scores are normalised over the frontier by softmax;
 * the node mass w_i is the mean over the G heads; the kept set is the
 * shortest prefix, in (w descending, node id ascending) order, whose mass
 * reaches p times the frontier total (everything when p >= 1); the next
 * frontier is the kept nodes' children.  The G heads of a KV head share one
 * kept set.  On return *kept views the level-1 kept chunk ids of each unit.
 * q: [B][Hq][d] in the tree dtype.  0 < p; p >= 1 keeps every node.
 * Errors: ZHA_ERR_INVALID (p <= 0 or not finite, null pointer, no prior
 * zha_build), ZHA_ERR_HIP. */
ZHA_API zha_status zha_route(zha_tree_t tree, const void* q, float p, float scale,
                     zha_kept* kept, hipStream_t stream);

/* zha_route with a routing mode.  ZHA_ROUTE_GROUP is zha_route.  With
 * ZHA_ROUTE_PER_HEAD (tree created with per_head_routes) every routing unit
 * is one (sequence, query head): its frontier, softmax, top-p cut and kept
 * set are that head's alone; *kept then views [B*Hq] counts and [B*Hq][cap]
 * ids, and zha_attend gives every head its own attention set.
 * Errors: as zha_route, and ZHA_ERR_INVALID for a per-head route on a tree
 * created without per_head_routes or for an unknown mode. */
ZHA_API zha_status zha_route_ex(zha_tree_t tree, const void* q, float p, float scale, zha_route_mode mode,
                        zha_kept* kept, hipStream_t stream);

/* Routes a block of Tq = n_queries consecutive queries of every sequence,
 * each query on its own, as a decode query is routed: the queries of a
 * prefill chunk or of a speculative verification step.  Every query descends
 * the tree from the top ([aitop] abstract: later queries traverse the tree top
 * down; [flux] "树形索引是怎么搭的": routing plus final attention per query grows
 * sublinearly with length, so attention over a whole sequence is
 * subquadratic).  The tree holds the N_b tokens before the block (the block's
 * own keys are not in it); query t of sequence b stands at position N_b + t.
 * q: [B][Tq][Hq][d] in the tree dtype.  Routing units are numbered
 * ((b * Tq + t) * Hkv + KV head) * hr + head, hr = 1 (ZHA_ROUTE_GROUP) or G
 * (ZHA_ROUTE_PER_HEAD); *kept views B*Tq*Hkv*hr counts and id rows.  A unit's
 * kept set is the one zha_route_ex would give that query alone.
 * Errors: as zha_route_ex; ZHA_ERR_INVALID for n_queries < 1;
 * ZHA_ERR_CAPACITY for n_queries above the tree's max_queries. */
ZHA_API zha_status zha_route_multi(zha_tree_t tree, const void* q, int32_t n_queries, float p, float scale,
                           zha_route_mode mode, zha_kept* kept, hipStream_t stream);

/* Device-side health of a tree.  The ordered compaction of a large level chains
 * its workgroups' kept counts with a decoupled look-back whose waits are bounded;
 * a wait that gives up (never expected: every workgroup it waits on has been
 * dispatched before it) marks the tree, and the kept lists of that route are then
 * not valid.  zha_tree_check synchronises the stream (unlike every other entry
 * point), reads the mark and clears it: ZHA_OK when no wait has given up since
 * the tree was created or last checked, ZHA_ERR_DEVICE otherwise.
 * Errors: ZHA_ERR_INVALID (null tree), ZHA_ERR_HIP. */
ZHA_API zha_status zha_tree_check(zha_tree_t tree, hipStream_t stream);

/* Exact attention of each query head over S = {token 0} U (tokens of the
 * kept chunks) U [Nc, N), S a set ([wqu] "How does top-p routing pick
 * tokens?": the first token is always kept; the trailing partial chunk is not
 * in the tree and is always read).  out_h = sum_{t in S} softmax_S(scale *
 * q_h.k_t) v_t and lse_h = log sum_{t in S} exp(scale * q_h.k_t), computed
 * in float32 from the stored K and V.  kept: the view returned by zha_route
 * on this tree.  Errors: ZHA_ERR_INVALID (also when the last route was a
 * zha_route_multi, or when zha_build or zha_append changed the tree after the
 * last route: the kept list no longer describes the cache), ZHA_ERR_HIP. */
ZHA_API zha_status zha_attend(zha_tree_t tree, const void* q, const void* K, const void* V,
                      const zha_kept* kept, float scale, float* out, float* lse,
                      hipStream_t stream);

/* Exact attention of a block of queries routed by zha_route_multi.  Query t
 * of sequence b attends S = {token 0} U (tokens of its kept chunks) U
 * [Nc_b, N_b + t + 1): besides the partial chunk, the block's rows up to its
 * own position, causally.  Rows N_b .. N_b + Tq - 1 of K and V hold the
 * block's keys and values (written there by the caller; zha_append adds them
 * to the tree afterwards).  q: [B][Tq][Hq][d]; out: [B][Tq][Hq][d] float32;
 * lse: [B][Tq][Hq] float32; same formulas as zha_attend.
 * Errors: ZHA_ERR_INVALID (kept is not the view of this tree's last route, that
 * route was not a zha_route_multi of n_queries queries, or the tree was built or
 * appended to after it), ZHA_ERR_CAPACITY
 * (N_b + n_queries > max_tokens for some b), ZHA_ERR_HIP. */
ZHA_API zha_status zha_attend_multi(zha_tree_t tree, const void* q, int32_t n_queries, const void* K,
                            const void* V, const zha_kept* kept, float scale, float* out, float* lse,
                            hipStream_t stream);

/* Dense decode attention over [0, N_b), the comparison baseline.  Same
 * layouts as zha_attend.  workspace: device scratch of at least
 * zha_dense_workspace_bytes(...) bytes, owned by the caller.
 * Errors: ZHA_ERR_INVALID, ZHA_ERR_CAPACITY, ZHA_ERR_UNSUPPORTED, ZHA_ERR_HIP. */
ZHA_API zha_status zha_dense_decode(const void* q, const void* K, const void* V,
                            const int32_t* seq_lens /* host [B] */,
                            int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, int64_t max_tokens, zha_dtype dtype,
                            float scale, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
ZHA_API size_t zha_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                 int32_t head_dim, int64_t max_tokens);

/* zha_dense_decode for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same kernels and
 * results, with the split-K partials in a fixed array of ZHA_DENSE_SCRATCH_BYTES bytes that
 * the library holds on each GPU it runs on until the process ends (its device address is
 * taken on the first call on that GPU).  No device memory is allocated or freed by any
 * call.  Shapes whose partials need more than the array
 * (zha_dense_workspace_bytes(...) > ZHA_DENSE_SCRATCH_BYTES) are rejected before anything
 * is enqueued.  Every call on one GPU uses the same array: calls that overlap on a GPU
 * (other streams, other host threads) race and must be serialised by the caller.
 * Errors: as zha_dense_decode; ZHA_ERR_CAPACITY also for shapes beyond the array;
 * ZHA_ERR_HIP when the array's address cannot be obtained. */
#define ZHA_DENSE_SCRATCH_BYTES ((size_t)8 << 20)
ZHA_API zha_status zha_dense_decode_noalloc(const void* q, const void* K, const void* V,
                                    const int32_t* seq_lens /* host [B] */,
                                    int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                    int32_t head_dim, int64_t max_tokens, zha_dtype dtype,
                                    float scale, float* out, float* lse, hipStream_t stream);

/* ---- inspection (tests and benchmarks) -------------------------------- */

/* Node capacity of a level (per unit): ceil(C*floor(max_tokens/C) / C^level). */
ZHA_API zha_status zha_tree_level_capacity(zha_tree_t tree, int32_t level, int64_t* nodes);

/* Copies level `level` (1..L) of the tree: m_out [B*Hkv][cap][R][d] in the
 * tree dtype and b_out [B*Hkv][cap][R] float32 (cap from
 * zha_tree_level_capacity).  With fp8 or fp4 summaries m_out receives the
 * decoded m~ = code * 2^e, exact in bf16.  Device buffers owned by the caller. */
ZHA_API zha_status zha_tree_copy_level(zha_tree_t tree, int32_t level, void* m_out, float* b_out,
                               hipStream_t stream);

/* Copies the scales 2^e of level `level` of a tree with low-precision
 * summaries: fp8, one per row, scale_out [B*Hkv][cap][R] float32; fp4, one per
 * block of 32 values, scale_out [B*Hkv][cap][R][d/32] float32.  A device
 * buffer owned by the caller.
 * Errors: ZHA_ERR_INVALID (null pointer, level out of range, native tree). */
ZHA_API zha_status zha_tree_copy_scales(zha_tree_t tree, int32_t level, float* scale_out, hipStream_t stream);

/* Copies the last route's result at `level`, per routing unit (RU = B*Hkv after
 * a group route, B*Hq after a per-head route): frontier_counts [RU],
 * kept_counts [RU], kept_ids [RU][cap] (ascending).  The frontier of level L is
 * every level-L node; the frontier of level l < L is the children of the kept
 * set of level l + 1.  Device buffers owned by the caller. */
ZHA_API zha_status zha_route_copy_level(zha_tree_t tree, int32_t level, int32_t* frontier_counts,
                                int32_t* kept_counts, int32_t* kept_ids, hipStream_t stream);

/* Per-kernel timing.  With kernel_mask != 0 the tree records a HIP event pair
 * on the stream around each launch whose kernel code k (ZHA_K_*) has bit k set
 * in kernel_mask and whose level l (0 for kernels without one) has bit l set in
 * level_mask; ZHA_TIMING_ALL selects every kernel or every level.  kernel_mask 0
 * turns timing off; changing the masks keeps what is already recorded.  After
 * the caller has synchronised the stream, zha_timing_read returns for each
 * recorded launch its kernel code, its level and its duration in ms, and
 * clears the record.  At most 256 launches are kept between reads; later ones
 * are not recorded.  The events only measure time (they are recorded without a
 * system-scope fence).  Not for use under stream capture. */
enum { ZHA_K_BUILD = 1, ZHA_K_APPEND = 2, ZHA_K_SCORE = 3, ZHA_K_SELECT = 4,
       ZHA_K_ATTEND = 5, ZHA_K_MERGE = 6, ZHA_K_MASS = 7, ZHA_K_COMPACT = 8 };
#define ZHA_TIMING_ALL (-1)
ZHA_API zha_status zha_timing_enable(zha_tree_t tree, int32_t kernel_mask, int32_t level_mask);
ZHA_API zha_status zha_timing_read(zha_tree_t tree, int32_t* kernels, int32_t* levels, float* ms,
                           int32_t max_entries, int32_t* n_entries);

/* Copy kernel of known size, used to calibrate hardware byte counters:
 * dst[i] = src[i] for n 16-byte elements (both device, 16-byte aligned). */
ZHA_API zha_status zha_calibration_copy(void* dst, const void* src, int64_t n16, hipStream_t stream);

ZHA_API const char* zha_status_str(zha_status status);

/* Text of the last HIP failure that made an entry point return ZHA_ERR_HIP on
 * the calling thread (empty when none); owned by the library. */
ZHA_API const char* zha_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZHA_H */
