/*
 * magicpig.h -- C ABI of the MI355X (gfx950) SimHash-sampled decode-attention
 * library (libmagicpig.so).
 *
 * The method is MagicPIG ("MagicPIG: LSH Sampling for Efficient LLM
 * Generation", arXiv 2410.16179v2).  One decode step of one attention layer
 * estimates o = softmax(q K^T / sqrt(d)) V (Section 2.1, Equation 1) from a
 * sampled subset S of the keys:
 *
 *   codes   every key k_i is centred by the key mean mu (Section 4.3 "Data
 *           pre-processing") and hashed by SimHash into L tables of K sign
 *           bits each (Section 2.2; Section 4.3 "Hash function selection");
 *   S       key i is sampled for a query when their codes agree in at least
 *           two of the L tables (Section 4.3, Equation 10);
 *   weight  each sampled key is weighted by exp(q.k_i/sqrt(d)) / P_i with
 *           P_i = 1 - (1-p)^L - L p (1-p)^(L-1), p = (1 - theta_i/pi)^K
 *           (Equations 10 and 11);
 *   output  the self-normalised estimate sum_S w_i v_i / sum_S w_i
 *           (Equation 9; Algorithm 1).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer is a DEVICE pointer on the current HIP device.  The caller
 *    allocates and owns every buffer; the library never allocates, frees or
 *    keeps pointers after a call returns, and keeps no global state, so calls
 *    on different streams are independent when their workspaces differ.  The
 *    one exception is mp_decode_step_static (at the end of this file), whose
 *    workspace is a fixed device array of the library, shared by its calls.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *    work is enqueued on it; nothing synchronises the host.  Results are valid
 *    once the stream has reached the point after the call.
 *  - Arguments are validated before anything is enqueued: a call that
 *    returns an error has written nothing.  No call aborts or prints.
 *  - The kernels move data in 16-byte vectors: the K/V caches, new key and
 *    value rows, queries, codes, kmean, the packed projection, out and the
 *    workspace must start on a 16-byte boundary (every hipMalloc and torch
 *    allocation does); a misaligned one is MP_ERR_ARG.  qcodes, lse, idx and
 *    count need only their element alignment.
 *  - Shapes: d (head dimension) must be 128.  0 <= K <= 16 bits per table,
 *    2 <= L <= 512 tables, K*L <= 4096.  Query heads per KV head
 *    G = Hq / Hkv must divide exactly and be at most 8.  Cache capacities
 *    `cap` must be multiples of 8 (16-byte code rows).  Units U = B * Hkv
 *    at most 65535; for the decode U * ceil(cap / 512) at most 2^23 and
 *    cap below 2^26 (MP_ERR_UNSUPPORTED otherwise).
 *  - Element types: MP_BF16 (bfloat16) or MP_F32 (float32) for keys, values
 *    and queries; codes are uint16; means, outputs and lse are float32.
 *  - Layouts (row-major, innermost last):
 *      K, V cache    [U][cap][d]     U = B * Hkv units (batch x KV head)
 *      codes         [U][L][cap]     table-major: code of table l of key i
 *                                    at codes[u][l][i]; bit b of table l is
 *                                    projection column l*K + b (LSB first)
 *      kmean         [U][d]          float32 key mean per unit
 *      q             [B][Hq][d]      query head h reads KV head h / G
 *      qcodes        [B][Hq][L]
 *      out           [B][Hq][d]      float32
 *      lse, count    [B][Hq]
 *      idx           [B][Hq][cap]    int32, ascending sampled key indices
 */
#ifndef MAGICPIG_H
#define MAGICPIG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
#define MP_OK 0
#define MP_ERR_ARG (-1)         /* null, misaligned or inconsistent argument */
#define MP_ERR_UNSUPPORTED (-2) /* shape outside the supported set          */
#define MP_ERR_CAPACITY (-3)    /* n >= cap on append, or n > cap           */
#define MP_ERR_WORKSPACE (-4)   /* workspace missing or smaller than needed */
#define MP_ERR_HIP (-5)         /* a HIP launch failed                      */
#define MP_ERR_SCRATCH (-6)     /* shape needs more than the static scratch  */

/* Element types of keys, values and queries. */
#define MP_BF16 0
#define MP_F32 1

/* Human-readable text for a status code (static storage, never NULL). */
const char *mp_strerror(int status);

/* Library ABI version (incremented on incompatible changes). */
int mp_version(void);

/*
 * Projection packing.  W is Algorithm 1's random projector matrix
 * W in R^{d x (K*L)} (Section 4.3 "Hash function selection"): float32,
 * row-major [d][K*L], column l*K + b being hyperplane b of table l.  It is
 * rounded to bf16 (round to nearest even) and rearranged into the operand
 * order of the encoder's matrix-core tiles (8 KB per tile of floor(32/K)
 * whole tables).  Wp receives mp_proj_bytes(d,K,L) bytes.  Both pointers are device pointers.  One packed W serves every
 * unit of a layer (the paper shares projectors across heads, Section 4.4).
 * Errors: MP_ERR_ARG (null pointers), MP_ERR_UNSUPPORTED (d, K, L limits).
 */
size_t mp_proj_bytes(int d, int K, int L);
int mp_proj_pack(const float *W, int d, int K, int L, void *Wp, void *stream);

/*
 * Code-store build (Section 4.3 "Data pre-processing" and "Hash function
 * selection"; the hash-table construction that the paper overlaps with
 * prefill, authors' reply to Q2 on page 3).  For each unit u < U:
 *   kmean[u] = fp32( (1/n) sum_{i<n} K[u][i] )  (fp64 accumulation),
 *   x_i      = bf16( fp32(K[u][i]) - kmean[u] ),
 *   bit_j    = ( x_i . bf16(W[:, j]) > 0 ),  code_l = sum_b bit_{l*K+b} << b,
 * written to codes[u][l][i] for i < n (columns >= n are not touched).  The
 * mean is frozen: later appends reuse it.
 *   Kc     [U][cap][d] keys (kv_dtype), first n rows read
 *   Wp     packed projections from mp_proj_pack
 *   kmean  out [U][d];  codes out [U][L][cap]
 *   ws     device workspace of at least mp_build_ws_bytes(U, n, d) bytes
 * Errors: MP_ERR_ARG, MP_ERR_UNSUPPORTED, MP_ERR_CAPACITY (n > cap or n < 1),
 * MP_ERR_WORKSPACE, MP_ERR_HIP.
 */
size_t mp_build_ws_bytes(int64_t U, int64_t n, int d);
int mp_build_codes(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, int d, const void *Wp, int K,
                   int L, float *kmean, uint16_t *codes, void *ws, size_t ws_bytes, void *stream);

/*
 * Append one decoded token per unit (Algorithm 1 keeps encoding new keys with
 * the same projections; the mean stays frozen at its build value).
 * Writes Kc[u][n] = k_new[u], Vc[u][n] = v_new[u] and the L codes of
 * bf16(k_new[u] - kmean[u]) at codes[u][l][n].  The caller then uses n + 1.
 *   k_new, v_new  [U][d] (kv_dtype);  Kc, Vc [U][cap][d];  codes [U][L][cap]
 * Errors: MP_ERR_ARG, MP_ERR_UNSUPPORTED, MP_ERR_CAPACITY (n >= cap),
 * MP_ERR_HIP.
 */
int mp_append(const void *k_new, const void *v_new, void *Kc, void *Vc, int kv_dtype, int64_t U, int64_t n,
              int64_t cap, int d, const float *kmean, const void *Wp, int K, int L, uint16_t *codes, void *stream);

/*
 * The lift of Section 4.2, Equation 8, as an option (the pages describe it
 * and do not use it, Section 5.1): r = max_i |x_i|, keys [x_i,
 * sqrt(r^2 - |x_i|^2)], queries [q, 0], so that the angle the hash preserves
 * follows the inner product.  It applies to the vectors that are hashed,
 * x_i = bf16(fp32(K[u][i]) - kmean[u]); r (rlift[u], fp32) is the largest
 * |x_i| of the build keys (fp64 sums) and is frozen with the mean; a key's
 * extra coordinate is e = bf16(fp32(sqrt(max(0, r^2 - |x|^2)))) (an appended
 * key longer than r gets 0), and bit j = (x . bf16(W[:d, j]) +
 * e bf16(W[d][j]) > 0).
 *   mp_proj_pack_lift: W is [d + 1][K*L] float32; Wp receives
 *     mp_proj_bytes_lift(d, K, L) bytes: the packed first d rows (as
 *     mp_proj_pack, so Wp also serves the query encoders) followed by the
 *     extra row.
 *   mp_build_codes_lift: as mp_build_codes, plus rlift out [U] float32.
 *   mp_append_lift: as mp_append, with the frozen rlift [U].
 *   mp_decode_attn_lift: as mp_decode_attn for keys hashed lifted; the
 *     sampling angle is the one between [q, 0] and the lifted key, whose
 *     norm is r: cos = q.(K_i - kmean) / (|q| rlift[u]) (rlift [B*Hkv]).
 * K >= 1 (MP_ERR_UNSUPPORTED otherwise); other errors as the unlifted calls.
 */
size_t mp_proj_bytes_lift(int d, int K, int L);
int mp_proj_pack_lift(const float *W, int d, int K, int L, void *Wp, void *stream);
int mp_build_codes_lift(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, int d, const void *Wp, int K,
                        int L, float *kmean, float *rlift, uint16_t *codes, void *ws, size_t ws_bytes, void *stream);
int mp_append_lift(const void *k_new, const void *v_new, void *Kc, void *Vc, int kv_dtype, int64_t U, int64_t n,
                   int64_t cap, int d, const float *kmean, const float *rlift, const void *Wp, int K, int L,
                   uint16_t *codes, void *stream);
int mp_decode_attn_lift(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                        const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                        const float *kmean, const float *rlift, const void *Wp, int B, int Hq, int Hkv, int64_t n,
                        int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                        const uint16_t *qcodes_in, uint16_t *qcodes_out, float *out, float *lse, int32_t *idx,
                        int32_t *count, void *ws, size_t ws_bytes, void *stream);

/*
 * Bit-plane index of the code store: the same codes, packed as K bit planes
 * per table (K bits per key and table instead of 16), so the collision scan
 * reads K/16 of the bytes.  Layout [U][ceil(cap/512)][K][L][16] uint32: word
 * j of row (b, l) of tile t holds bit b of codes[u][l][i] for keys
 * i = 512 t + 32 j + e at bit e (e < 32); a tile's rows are contiguous.
 * mp_build_planes fills tiles [n0/512, n1/512) of every unit from codes
 * (their keys must have been written); n0 and n1 multiples of 512 with
 * 0 <= n0 <= n1 <= cap.  Appends do not update it: a decode scans the
 * planes only for tiles below its n_planes and the 16-bit codes elsewhere,
 * so the caller rebuilds the newest tile once it is full.
 *   codes  [U][L][cap] (mp_build_codes);  planes out, mp_planes_bytes bytes
 * Errors: MP_ERR_ARG (null or misaligned pointers, n0 / n1 not multiples of
 * 512 or out of range, K = 0), MP_ERR_UNSUPPORTED (shape), MP_ERR_HIP.
 */
size_t mp_planes_bytes(int64_t U, int64_t cap, int K, int L);
int mp_build_planes(const uint16_t *codes, int64_t U, int64_t n0, int64_t n1, int64_t cap, int K, int L,
                    uint32_t *planes, void *stream);

/*
 * Bucketed hash tables of the code store: the L hash tables of 2^K buckets
 * that the method builds from the keys' codes (Section 2.2 "Locality
 * sensitive hashing"; Section 4.4, the retrieval step that looks the query's
 * codes up in pre-built tables; built per layer, authors' reply to Q2 on
 * page 3).  A decode that uses them reads only the query's L buckets per
 * head instead of every key's codes; the sampled sets are the same, since a
 * key is in the query's bucket of table l exactly when codes[u][l][i] equals
 * the query's code of table l.
 * Layout (one buffer of mp_buckets_bytes(U, cap, K, L) bytes): keys are cut
 * into chunks of MP_BUCKET_CHUNK (8192); per (unit, table, chunk) a CSR of
 * the chunk's keys ordered by code --
 *   off   [U][L][2^K][ceil(cap/8192)] uint32 at the buffer's start: word
 *         (u, l, c, r) = start | count << 16, bucket c of chunk r holds
 *         entries start .. start + count - 1 (a bucket's words for all
 *         chunks are adjacent: a lookup reads one line of them per table);
 *   keys  [U][L][cap] uint16, starting at the next 256-byte boundary:
 *         entry j of chunk r of table l is keys[u][l][8192 r + j], the key's
 *         offset from the chunk's first key (the order inside a bucket is
 *         not fixed).
 * mp_build_buckets (re)builds the chunks [n0/8192, ceil(n1/8192)) from the
 * codes of keys below n1 (written by mp_build_codes / mp_append); n0 a
 * multiple of 8192, n1 a multiple of 512, 0 <= n0 <= n1 <= cap.  Appends do
 * not update it: a decode uses the buckets for the 512-key tiles below its
 * n_buckets and the codes (or planes) above, so the caller rebuilds the
 * newest chunk once a tile has filled.  1 <= K <= 12.
 * Errors: MP_ERR_ARG (null or misaligned pointers, n0 / n1 out of range),
 * MP_ERR_UNSUPPORTED (shape), MP_ERR_WORKSPACE (buffer smaller than
 * mp_buckets_bytes), MP_ERR_HIP.
 */
#define MP_BUCKET_CHUNK 8192
size_t mp_buckets_bytes(int64_t U, int64_t cap, int K, int L);
int mp_build_buckets(const uint16_t *codes, int64_t U, int64_t n0, int64_t n1, int64_t cap, int K, int L,
                     void *buckets, size_t buckets_bytes, void *stream);

/*
 * Query encoding (Algorithm 1, "Compute hash code for new query"):
 * qcodes[r][l] = code of table l of y_r = bf16(q[r]); queries are NOT
 * centred (centring shifts keys only; softmax is translation invariant).
 *   q       [nq][d] (q_dtype);  qcodes out [nq][L]
 * Errors: MP_ERR_ARG, MP_ERR_UNSUPPORTED, MP_ERR_HIP.
 */
int mp_encode_queries(const void *q, int q_dtype, int64_t nq, int d, const void *Wp, int K, int L, uint16_t *qcodes,
                      void *stream);

/*
 * Sampled decode attention of one layer (Algorithm 1 for every query head;
 * Equations 9-11).  For query head h of batch b (KV unit u = b*Hkv + h/G):
 *   S_h   = { i < n : #{l : codes[u][l][i] == qcode_h[l]} >= T }
 *           plus the forced ranges i < n_static_head and
 *           i >= n - n_static_tail (probability 1; Algorithm 1's static
 *           cache K_T, V_T and the authors' reply on sink tokens),
 *   cos_i = q_h.(K_i - kmean_u) / (|q_h| |K_i - kmean_u|),
 *   lnP_i = ln sum_{j>=T} C(L,j) p^j (1-p)^(L-j), p = (1 - acos(cos_i)/pi)^K
 *           (for the pages' threshold T = 2: ln(1 - (1-p)^L - L p (1-p)^(L-1)),
 *           Equation 10),
 *   s_i   = q_h.K_i / sqrt(d) - lnP_i,
 *   out   = sum_{S_h} e^{s_i} V_i / sum_{S_h} e^{s_i},  lse = ln sum e^{s_i}.
 * T is the collision threshold, 1 <= T <= L (MP_ERR_UNSUPPORTED otherwise);
 * the pages use T = 2 (a key colliding with the query in at least two
 * tables, Section 4.3), and the benchmarked workloads do too.
 * All G query heads of a KV head share one pass over its codes; each head
 * keeps its own set and probabilities.  An empty set gives out = 0,
 * lse = -inf, count = 0.
 *   q          [B][Hq][d] (kv_dtype)
 *   Kc, Vc     [B*Hkv][cap][d];  codes [B*Hkv][L][cap];  kmean [B*Hkv][d]
 *   planes     nullable bit-plane index (mp_build_planes) valid for tiles
 *              below n_planes (a multiple of 512, 0 <= n_planes <= n): with
 *              T = 2 those tiles are scanned from it; the sets and outputs
 *              are the same as from codes.  n_planes is ignored when planes
 *              is NULL.
 *   buckets    nullable bucketed tables (mp_build_buckets) valid for keys
 *              below n_buckets (a multiple of 512, 0 <= n_buckets <= n):
 *              with T = 2 the tiles below n_buckets take their sampled keys
 *              from the query's buckets (one more kernel, before the
 *              sampling kernel) and are not scanned; the sets and outputs
 *              are the same.  Tiles below n_buckets take precedence over
 *              planes.  Ignored for other thresholds.
 *   Wp         packed projections (read only when qcodes_in is NULL)
 *   qcodes_in  nullable [B][Hq][L]: use these query codes instead of
 *              encoding q
 *   qcodes_out nullable [B][Hq][L]: receives the codes when q is encoded here
 *   out        [B][Hq][d] float32;  lse nullable [B][Hq] float32
 *   idx        nullable [B][Hq][cap] int32: the sampled indices, ascending
 *   count      nullable [B][Hq] int32: |S_h|
 *   ws         device workspace of mp_decode_ws_bytes(B, Hq, Hkv, cap, d, L)
 *              bytes (the same size for every n <= cap)
 * Errors: MP_ERR_ARG, MP_ERR_UNSUPPORTED, MP_ERR_CAPACITY (n < 0 or n > cap; n = 0 is
 * an empty cache),
 * MP_ERR_WORKSPACE, MP_ERR_HIP.
 */
size_t mp_decode_ws_bytes(int B, int Hq, int Hkv, int64_t cap, int d, int L);
int mp_decode_attn(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                   const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                   const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n, int64_t cap, int d, int K,
                   int L, int T, int64_t n_static_head, int64_t n_static_tail, const uint16_t *qcodes_in,
                   uint16_t *qcodes_out, float *out, float *lse, int32_t *idx, int32_t *count, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * The two stages of mp_decode_attn, callable separately (one kernel each),
 * for callers that schedule or time them apart.  mp_decode_sample runs the
 * collision scan, the weighting and the split attention (Equations 9-11
 * over key chunks) and leaves per-chunk partial results in ws;
 * mp_decode_merge combines them by log-sum-exp (the recursive-attention
 * merge of Section 4.4 "On-device cache") into out / lse / count / idx.
 * Both must see the same arguments and the same ws; want_idx must be
 * non-zero in mp_decode_sample when mp_decode_merge receives idx.
 * qcodes is required here ([B][Hq][L]).  mp_decode_merge takes the
 * sampling stage's kv_dtype, T and n_buckets (0 when it had no buckets):
 * with them it reads the partial records that stage filled, in the same
 * order as mp_decode_attn, whose results it then reproduces bit for bit.
 */
int mp_decode_sample(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                     const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                     const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                     int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail, int want_idx, void *ws,
                     size_t ws_bytes, void *stream);
int mp_decode_merge(int kv_dtype, int B, int Hq, int Hkv, int64_t n, int64_t cap, int d, int L, int T,
                    int64_t n_buckets, float *out, float *lse, int32_t *idx, int32_t *count, void *ws,
                    size_t ws_bytes, void *stream);

/*
 * One decode step of one layer in three launches: append the new token's key
 * and value to every unit and encode its key (as mp_append; skipped when
 * k_new is NULL), encode the queries (as mp_encode_queries, into ws) -- both
 * in one launch -- then sample and merge (as mp_decode_attn) over n + 1 keys
 * (n keys without an append).  Arguments as in mp_append and
 * mp_decode_attn; q codes are kept in ws.  The appended key is not added to
 * planes or buckets (n_planes, n_buckets <= n, the keys before the append).  sample_events is NULL or points
 * to two host hipEvent_t handles that are attached to the sampling kernel's
 * dispatch, so they record its own start and end (for callers that time it;
 * with no keys to decode there is no such kernel and both are recorded back to
 * back).
 * Errors: as mp_append and mp_decode_attn; MP_ERR_CAPACITY when appending
 * with n >= cap.
 */
int mp_decode_step(const void *k_new, const void *v_new, const void *q, void *Kc, void *Vc, int kv_dtype,
                   uint16_t *codes, const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                   const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                   int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail, float *out, float *lse,
                   int32_t *idx, int32_t *count, void *ws, size_t ws_bytes, void *sample_events, void *stream);

/*
 * mp_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Arguments, results and errors are those
 * of mp_decode_step without ws / ws_bytes; the workspace is instead a fixed
 * device array of MP_STATIC_SCRATCH_BYTES bytes inside the library, one per
 * GPU, held until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); its first call on a
 * device looks up that device's array.  Shapes whose workspace
 * (mp_decode_ws_bytes) exceeds MP_STATIC_SCRATCH_BYTES return
 * MP_ERR_SCRATCH before anything is enqueued.  Every call on one GPU uses
 * that GPU's array, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls that overlap on one GPU (other streams or
 * threads) race on it, so the caller serialises them, e.g. on one stream.
 */
#define MP_STATIC_SCRATCH_BYTES (32u << 20)
int mp_decode_step_static(const void *k_new, const void *v_new, const void *q, void *Kc, void *Vc, int kv_dtype,
                          uint16_t *codes, const uint32_t *planes, int64_t n_planes, const void *buckets,
                          int64_t n_buckets, const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n,
                          int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                          float *out, float *lse, int32_t *idx, int32_t *count, void *sample_events, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MAGICPIG_H */
