/*
 * pariskv.h -- C ABI of the MI355X (gfx950) ParisKV decode path.
 *
 * ParisKV ("ParisKV: Fast and Drift-Robust KV-Cache Retrieval for Long-Context
 * LLMs") keeps the full KV cache, encodes every key of the retrieval zone into
 * compact metadata (sign-pattern bucket ids, 4-bit sign+magnitude codes and a
 * calibration scale per subspace), and at every decode step retrieves the
 * top-k keys for the current query coarse-to-fine on the GPU before running
 * attention over sink + local + update buffer + the retrieved keys.
 *
 * Terms used below:
 *   d      head dimension (128)           B   subspaces (16, 32 or 8)  m  coordinates per subspace
 *                                                                        (8, 4 or 16; B * m = d)
 *   unit   one (batch, kv head) sequence  G   query heads per kv head (grouped-query attention)
 *   cap    capacity in tokens per unit    N   tokens currently held per unit
 *
 * Memory layouts (row-major, innermost last):
 *   K / V store   [batch][n_kv_heads][cap][d]      kv_dtype, caller-owned
 *   q             [batch][n_q_heads][d]            kv_dtype; query head h belongs to kv head h / G
 *   k_new, v_new  [batch][n_kv_heads][d]           kv_dtype
 *   sel           [batch][n_kv_heads][top_k]       int32 token positions, ascending
 *   sel_n         [batch][n_kv_heads]              int32 number of valid entries of sel
 *   out           [batch][n_q_heads][d]            float32
 * All device pointers must be 16-byte aligned (checked: PK_ERR_INVALID); rows
 * are contiguous.
 *
 * Streams: every call that launches work takes a hipStream_t (passed as
 * void*, NULL = the null stream) and returns without synchronising.  Errors
 * found by host-side validation are returned before anything is launched and
 * leave the context unchanged.  A device fault surfaces as PK_ERR_HIP from a
 * later call.  A runtime call that fails inside the library (an allocation, a
 * launch) is reported only through the returned status: the library clears
 * the calling thread's HIP last-error state before returning, so the caller's
 * own later error checks do not see it.
 *
 * HIP graph capture: each call takes its launch decisions (grid sizes, window
 * bounds, the candidate count) on the host from the context's window, and a
 * captured call replays the decisions it was captured with.  Device state
 * carried between calls (the coarse-score histogram) is returned to zero by
 * the call that consumes it, so pk_retrieve and pk_sparse_attend on a static
 * context (no appends: the window does not move) can be captured once and
 * replayed with new query contents.  Calls that move the window
 * (pk_append_decode_keys, pk_decode_step) must be issued eagerly, one per
 * token.  The decode-path calls allocate nothing and never synchronise.  A
 * context is not thread-safe; calls on one context must be issued from one
 * host thread in order.
 */
#ifndef PARISKV_H
#define PARISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PK_OK = 0,
    PK_ERR_INVALID = -1,      /* bad argument or configuration                      */
    PK_ERR_NO_DEVICE = -2,    /* no usable gfx950 device                            */
    PK_ERR_OOM = -3,          /* device allocation failed                           */
    PK_ERR_CAPACITY = -4,     /* the token would exceed the context's capacity      */
    PK_ERR_HIP = -5,          /* a HIP runtime call failed (launch or earlier fault) */
    PK_ERR_UNSUPPORTED = -6   /* valid, but not a configuration this library builds */
} pk_status;

typedef enum { PK_F32 = 0, PK_BF16 = 1 } pk_dtype;

/* Where the caller's K/V store lives.  PK_MEM_HOST_MAPPED: pinned host memory
 * mapped into the device address space; attention then reads retrieved rows
 * over the host link, as in the page's UVA offloading. */
typedef enum { PK_MEM_DEVICE = 0, PK_MEM_HOST_MAPPED = 1 } pk_mem;

/* Method parameters.  ParisKV page: "Analytic centroids" (B, m), "Coarse
 * candidate generation" (rho, vote weights, candidate fraction), "Sliding-window
 * update mechanism" (zones).  Supported: head_dim 128 and (n_sub, sub_dim) =
 * (16, 8), (32, 4) or (8, 16); n_sub * sub_dim != head_dim is PK_ERR_INVALID,
 * other widths PK_ERR_UNSUPPORTED.  Every width keeps the 16 sign bytes of the
 * rotated key as its bucket ids:
 *   m = 8   one id per byte; the vote table has a 256-entry byte row per subspace;
 *   m = 4   the 2^4 sign-pattern centroids give 4-bit ids, two per id byte, the
 *           vote table's byte row i sums subspaces 2i and 2i + 1, and
 *           G * max(weight) <= 127;
 *   m = 16  the 16-bit id of subspace b is the little-endian word at bytes 2b,
 *           2b + 1; of its 65536 centroids only the G * rho voted ones have a
 *           vote, kept per subspace in a 256-slot hash table (see PK_DBG_LUT),
 *           and G * max(weight) <= 255. */
typedef struct {
    int32_t head_dim;          /* d = 128                                             */
    int32_t n_sub;             /* B = 16 (or 32, or 8)                                */
    int32_t sub_dim;           /* m = 8: 256 sign-pattern centroids per subspace;     */
                               /* m = 4: 16 of them; m = 16: 65536                    */
    int32_t rho;               /* centroids picked per subspace and query head, 1..8  */
    uint8_t vote_weight[8];    /* vote of a rank-r pick (r = 0 is the best), 1..255   */
    int32_t coarse_permille;   /* candidates kept = max(top_k, ceil(p * N_r / 1000)), capped at N_r */
    int32_t top_k;             /* keys retrieved per unit, >= 1                       */
    int32_t n_sink;            /* first tokens always attended                        */
    int32_t n_local;           /* most recent tokens always attended                  */
    int32_t buf_tokens;        /* update buffer U (0 = static context, no appends)    */
    uint64_t sign_bits[2];     /* SRHT diagonal: D_jj = -1 where bit j is set         */
    int32_t codebook;          /* magnitude codebook: 0 = Lloyd-Max (pk_codebook), 1 = */
                               /* equal-probability bins (pk_codebook_quantile)       */
} pk_config;

typedef struct pk_ctx pk_ctx;  /* opaque; owned by the library */

/* Create a context over the caller's K/V store.
 * Owns: the per-key metadata (16 B of bucket ids and a record of codes and
 * scales per token: 64 B of 4-bit codes + 4 B per subspace, so 128 B for m = 8,
 * 192 B for m = 4 and 96 B for m = 16), the window counters and all scratch.  The caller
 * keeps ownership of k_store / v_store, which must outlive the context.
 * Requires batch * n_kv_heads <= 65535 (else PK_ERR_UNSUPPORTED) and
 * n_q_heads = G * n_kv_heads with G in {1, 2, 4, 8} (other G up to 16
 * are valid but PK_ERR_UNSUPPORTED), G * max(weight) <= 255 (m = 8, 16; 127 for m = 4), buf_tokens <=
 * n_local, capacity <= 2^24.  Allocates device memory and synchronises the device.
 * Errors: PK_ERR_INVALID, PK_ERR_UNSUPPORTED, PK_ERR_NO_DEVICE, PK_ERR_OOM. */
pk_status pk_create(const pk_config* cfg, int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                    int64_t capacity, pk_dtype kv_dtype, void* k_store, void* v_store,
                    pk_mem store_mem, pk_ctx** out);

/* Free the context (synchronises the device).  NULL is ignored. */
void pk_destroy(pk_ctx* ctx);

/* Prefill.  The caller has written n_tokens tokens of every unit into the
 * store.  Sets the window (sink = first n_sink tokens, local = last n_local,
 * retrieval in between, empty buffer) and encodes every retrieval-zone key:
 * SRHT rotation, bucket id per subspace, 4-bit code per coordinate, scale w
 * per subspace.  ParisKV page: "Normalization and rotation", "Coarse candidate
 * generation", "Quantization", "Calibration" (w is computed at prefill).
 * Errors: PK_ERR_INVALID (n_tokens < 1), PK_ERR_CAPACITY (n_tokens > cap). */
pk_status pk_encode_keys(pk_ctx* ctx, int64_t n_tokens, void* stream);

/* Decode append: write one new token per unit (device k_new / v_new) at
 * position N, into the update buffer.  If the previous step filled the buffer
 * (U tokens), first move the oldest local tokens into the retrieval zone and
 * encode them on the device, and promote the buffer to local.  ParisKV page:
 * "Sliding-window update mechanism".
 * Errors: PK_ERR_INVALID (buf_tokens == 0 or NULL input), PK_ERR_CAPACITY. */
pk_status pk_append_decode_keys(pk_ctx* ctx, const void* k_new, const void* v_new, void* stream);

/* Retrieval for the current queries q (device).  Per unit: rotate the G
 * queries, pick the top-rho centroids per subspace, score every retrieval-zone
 * key by its summed collision votes, keep the top candidates, rerank them with
 * the RSQ-IP estimate  sum_g ||q_g|| sum_b w_b <v_b, q~_b>  and write the top-k
 * positions to sel (ascending) and their count to sel_n.  Ties go to the lower
 * token position.  ParisKV page: "Coarse candidate generation",
 * "Candidate reranking (RSQ-IP)", "Estimation".
 * Errors: PK_ERR_INVALID (NULL pointer, or no prefill yet). */
pk_status pk_retrieve(pk_ctx* ctx, const void* q, int32_t* sel, int32_t* sel_n, void* stream);

/* Sparse GQA decode attention of q over sink + local + update buffer + the
 * sel_n[u] positions in sel (any positions of the retrieval zone, e.g. those
 * pk_retrieve wrote).  out = softmax(q k^T / sqrt(d)) V over that set, float32.
 * ParisKV page: "Problem definition" (attention over a top-k subset), "UVA
 * offloading" (retrieved rows may live in host memory).
 * Errors: PK_ERR_INVALID (NULL pointer, or no prefill yet). */
pk_status pk_sparse_attend(pk_ctx* ctx, const void* q, const int32_t* sel, const int32_t* sel_n,
                           float* out, void* stream);

/* Full attention over every stored token of each unit (no retrieval): the
 * dense GQA decode attention the sparse path replaces, kept as the comparison
 * baseline.  q device [batch][n_q][d] in the store dtype, out device float32
 * [batch][n_q][d]; the same split kernel and merge as pk_sparse_attend with
 * all n tokens as one zone.  The first call allocates its partial buffer
 * (units x ceil(n / 128) x G x 130 floats).  Device stores only.
 * ParisKV page, "Problem definition" (full attention reads every KV vector).
 * Errors: PK_ERR_INVALID (NULL pointer, no prefill), PK_ERR_UNSUPPORTED
 * (host-memory store, or more than 65535 x 128 tokens per unit), PK_ERR_OOM. */
pk_status pk_dense_attend(pk_ctx* ctx, const void* q, float* out, void* stream);

/* pk_dense_attend for callers that cannot allocate device memory during the
 * call (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): same arguments, layouts and results, but the split
 * partials go to a scratch array the library keeps in device memory (one per
 * GPU, pk_noalloc_scratch_bytes() = 64 MiB, held until the process ends;
 * its device address is looked up by pk_create) instead of a buffer allocated
 * on first use.  Calls no allocating routine.  All calls on one GPU share the
 * array: calls that overlap on one GPU (other streams, other contexts, other
 * host threads) race and must be ordered by the caller.  Each call rewrites
 * every partial it reads, so nothing carries over from an earlier call.
 * Errors: as pk_dense_attend, and PK_ERR_CAPACITY when the partials, batch *
 * n_q_heads * ceil(n / 128) * 130 floats (n = tokens held), exceed the array. */
pk_status pk_dense_attend_noalloc(pk_ctx* ctx, const void* q, float* out, void* stream);

/* Size in bytes of the scratch array used by pk_dense_attend_noalloc. */
size_t pk_noalloc_scratch_bytes(void);

/* Comparison coarse stage: replaces the analytic sign-pattern centroids of
 * every unit and subspace by 256 centroids fitted with k-means to the rotated
 * keys of positions [0, n_tokens) of the store (the keys a model holds after
 * prefill), the design the ParisKV page sets its data-independent centroids
 * against ("Problem definition"; "Drift-robust analytic centroids").  Call it
 * after writing the prefill K and before pk_encode_keys; from then on the
 * context's bucket ids (prefill and every later eviction) and the queries'
 * top-rho centroids use the fitted tables, and everything else is unchanged.
 * Fitting: init_pos device int32 [units][256] (positions < n_tokens, checked
 * on the host after a synchronising copy) give the initial centroids, the
 * normalised subspace vectors of those keys; then `iters` Lloyd rounds of
 * assignment (most similar centroid by the fp32 pairwise tree of the products
 * c_j x_j, ties to the lower index) and update (centroid = S / ||S||, S the
 * exact integer sum of the assigned vectors with coordinates rounded to
 * multiples of 2^-20; a centroid with no members keeps its value).  The first
 * call allocates the tables (units x 16 x 256 x 8 floats, and as many 64-bit
 * sums).
 * Errors: PK_ERR_INVALID (NULL, keys already encoded, n_tokens < 256, a
 * position out of range, iters outside 0..1000), PK_ERR_UNSUPPORTED (m != 8),
 * PK_ERR_CAPACITY, PK_ERR_OOM. */
pk_status pk_fit_centroids(pk_ctx* ctx, int64_t n_tokens, const int32_t* init_pos, int32_t iters,
                           void* stream);

/* One whole decode step: pk_append_decode_keys(k_new, v_new) followed by
 * pk_retrieve(q) and pk_sparse_attend(q) over the retrieved set, with the
 * append carried out by the retrieval's first kernel.  Same arguments,
 * layouts and results as the three calls in that order.
 * Errors: as pk_append_decode_keys; a PK_ERR_HIP leaves the context unusable. */
pk_status pk_decode_step(pk_ctx* ctx, const void* k_new, const void* v_new, const void* q,
                         int32_t* sel, int32_t* sel_n, float* out, void* stream);

/* Host only, no device needed.  The sign+3-bit magnitude codebook for sub_dim
 * m: the Lloyd-Max quantiser of |u_j| for u uniform on the unit sphere of R^m
 * (u_j^2 ~ Beta(1/2, (m-1)/2), the page's Beta prior).  levels[n_levels]
 * = fp32 levels, sq_thresholds[n_levels-1] = fp32(t^2) of the thresholds.
 * ParisKV page: "Quantization".  Errors: PK_ERR_INVALID (m < 2, n_levels != 8, NULL). */
pk_status pk_codebook(int32_t sub_dim, int32_t n_levels, float* levels, float* sq_thresholds);

/* Host only.  The other reading of the page's Beta-prior codebook: the same
 * law of |u_j|, cut into n_levels bins of equal probability (threshold l =
 * the l/n_levels quantile), each level the conditional mean of its bin.  Same
 * outputs and errors as pk_codebook.  ParisKV page: "Quantization". */
pk_status pk_codebook_quantile(int32_t sub_dim, int32_t n_levels, float* levels,
                               float* sq_thresholds);

/* Human-readable name of a status code (static string). */
const char* pk_status_string(pk_status s);

/* Current window of the context (same for every unit), host-side mirror. */
pk_status pk_get_window(const pk_ctx* ctx, int64_t* n_tokens, int64_t* sink_end, int64_t* r_end,
                        int64_t* buf);

/* Measurement reference, not part of the method: reads `bytes` bytes at `src`
 * (device memory, 16-byte aligned, a multiple of 16 bytes, at most 2^44) with a
 * plain streaming kernel (each 256-thread block one contiguous 32 KB piece,
 * eight 16-byte nontemporal loads per thread in flight), so that the path's
 * bandwidth can be set against this device's streaming-read rate.  *sink
 * (device, 4 bytes) is written only in the unlikely case that the checksum of
 * the data equals a fixed constant.  kernel_us: NULL, or a host float that
 * receives the kernel's duration in microseconds, timed by events attached to
 * the dispatch (the per-stage profile's timing); the call then waits for the
 * kernel.  Errors: PK_ERR_INVALID (NULL, misaligned or zero size), PK_ERR_HIP. */
pk_status pk_stream_read(const void* src, size_t bytes, uint32_t* sink, float* kernel_us,
                         void* stream);

/* Measurement reference, not part of the method: gathers `count` records of
 * `rec_bytes` bytes (a multiple of 16, at most 1024), record i being row
 * idx[i] of the array at `src` (device memory, 16-byte aligned, n_rows rows of
 * rec_bytes; idx device int32, values clamped to [0, n_rows) on the device),
 * 16 bytes per lane, so that the path's gather stages (the rerank's 128-byte
 * records, the attention's 256-byte K/V rows) can be set against this device's
 * random-gather rate for the same access pattern.  *sink (device, 4 bytes) is
 * written only in the unlikely case that the checksum equals a fixed constant.
 * kernel_us: as for pk_stream_read.
 * Errors: PK_ERR_INVALID (NULL, misaligned, sizes out of range), PK_ERR_HIP. */
pk_status pk_gather_read(const void* src, int64_t n_rows, int32_t rec_bytes, const int32_t* idx,
                         int64_t count, uint32_t* sink, float* kernel_us, void* stream);

/* Per-stage kernel timing.  While enabled, every kernel the context launches
 * is bracketed by HIP events recorded on the stream it runs on.
 * pk_profile_read synchronises those events and returns, per stage, the
 * summed duration in milliseconds and the number of launches since the last
 * enable (arrays of PK_STAGE_COUNT entries).  The coarse threshold is found
 * inside the rerank launch, so PK_STAGE_SELECT records no launches.
 * Errors: PK_ERR_INVALID. */
enum { PK_STAGE_ENCODE = 0, PK_STAGE_APPEND = 1, PK_STAGE_QPREP = 2, PK_STAGE_SCAN = 3,
       PK_STAGE_SELECT = 4, PK_STAGE_RERANK = 5, PK_STAGE_FINE = 6, PK_STAGE_ATTEND = 7,
       PK_STAGE_COMBINE = 8, PK_STAGE_COUNT = 9 };
pk_status pk_profile_enable(pk_ctx* ctx, int32_t on);
pk_status pk_profile_read(pk_ctx* ctx, double* ms, int64_t* launches);

/* Debug read-back for tests: copies an internal buffer to host memory and
 * synchronises the stream.  `bytes` must equal the size reported by
 * pk_debug_size for `what`.
 *   PK_DBG_IDS     uint8  [units][cap][16]          bucket ids (m = 4: subspace 2i in the low half of byte i;
 *                                                   m = 16: little-endian uint16 per subspace)
 *   PK_DBG_REC     uint8  [units][cap][64 + 4B]     64 B nibbles (coord 2i in low half of byte i) + float32 w[B]
 *   PK_DBG_LUT     uint8  [units][16][256]          vote of each id-byte value, last pk_retrieve (m = 4:
 *                                                   row i entry c = L[2i][c & 15] + L[2i+1][c >> 4]);
 *                  m = 16: uint32 [units][8][256]   per subspace a linear-probing hash table of the voted
 *                                                   centroids: vote << 16 | centroid, 0 = empty, home slot
 *                                                   ((c * 40503) & 0xffff) >> 8
 *   PK_DBG_SCORES  uint8  [units][cap]              min(coarse score, 255) of retrieval position sink_end + i
 *   PK_DBG_CAND    int32  [units][cmax]             candidate positions (ascending), first n_cand valid
 *   PK_DBG_EST     float  [units][cmax]             RSQ-IP estimate of each candidate
 *   PK_DBG_NCAND   int32  [units][4]                {threshold score, ties taken, n_cand, k_eff}
 *   PK_DBG_CENTROIDS float [units][B][256][8]       fitted centroids (after pk_fit_centroids only) */
enum { PK_DBG_IDS = 0, PK_DBG_REC = 1, PK_DBG_LUT = 2, PK_DBG_SCORES = 3, PK_DBG_CAND = 4,
       PK_DBG_EST = 5, PK_DBG_NCAND = 6, PK_DBG_CENTROIDS = 7 };
size_t pk_debug_size(const pk_ctx* ctx, int32_t what);
pk_status pk_debug_copy(pk_ctx* ctx, int32_t what, void* host_dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PARISKV_H */
