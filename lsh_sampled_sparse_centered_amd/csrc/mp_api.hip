// C ABI of libmagicpig.so: argument validation, workspace carving and kernel
// launches.  Every check runs before the first enqueue, so a call that
// returns an error has written nothing.
#include <atomic>
#include <mutex>

#include "magicpig.h"
#include "mp_internal.h"

using namespace mp;

namespace {

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

int check_shape(int d, int K, int L) {
  if (d != D) return MP_ERR_UNSUPPORTED;
  if (K < 0 || K > 16 || L < 2 || L > MAX_L || K * L > 4096) return MP_ERR_UNSUPPORTED;
  return MP_OK;
}

int check_dtype(int t) { return (t == MP_BF16 || t == MP_F32) ? MP_OK : MP_ERR_ARG; }

int check_heads(int B, int Hq, int Hkv) {
  if (B < 1 || Hq < 1 || Hkv < 1) return MP_ERR_ARG;
  if (Hq % Hkv != 0) return MP_ERR_ARG;
  if (Hq / Hkv > MAX_G) return MP_ERR_UNSUPPORTED;
  if ((int64_t)B * Hkv > 65535) return MP_ERR_UNSUPPORTED;  // grid.y of the key-mean kernels
  return MP_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MP_OK : MP_ERR_HIP; }

// The kernels move rows, code words, means and partials in 16-byte vectors.
// Null passes (each entry point checks the pointers it requires separately).
bool a16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
template <typename... P>
bool all_a16(const P *...p) {
  return (a16(p) && ...);
}

}  // namespace

extern "C" {

const char *mp_strerror(int status) {
  switch (status) {
    case MP_OK: return "success";
    case MP_ERR_ARG: return "invalid argument (null or misaligned pointer, or inconsistent sizes)";
    case MP_ERR_UNSUPPORTED: return "unsupported shape (need d = 128, 0 <= K <= 16, 2 <= L <= 512, K*L <= 4096, "
                                    "Hq/Hkv <= 8, B*Hkv <= 65535, B*Hkv*ceil(cap/512) <= 2^23)";
    case MP_ERR_CAPACITY: return "capacity exceeded (n > cap, n < 1 for a build, n < 0 for a decode, or n >= cap on an append)";
    case MP_ERR_WORKSPACE: return "workspace missing or too small";
    case MP_ERR_HIP: return "HIP kernel launch failed";
    case MP_ERR_SCRATCH: return "workspace of this shape exceeds the static scratch of mp_decode_step_static "
                                "(MP_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int mp_version(void) { return 3; }

size_t mp_proj_bytes(int d, int K, int L) {
  if (check_shape(d, K, L) != MP_OK) return 0;
  return (size_t)enc_ntiles(K, L) * KSTEPS * 64 * 16;
}

int mp_proj_pack(const float *W, int d, int K, int L, void *Wp, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if (K > 0 && (!W || !Wp)) return MP_ERR_ARG;
  if (!all_a16(Wp)) return MP_ERR_ARG;
  return hip_status(launch_proj_pack(W, K, L, Wp, as_stream(stream)));
}

size_t mp_build_ws_bytes(int64_t U, int64_t n, int d) {
  if (U < 1 || n < 1 || d != D) return 0;
  return (size_t)U * kmean_parts(n) * D * sizeof(double);
}

int mp_build_codes(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, int d, const void *Wp, int K,
                   int L, float *kmean, uint16_t *codes, void *ws, size_t ws_bytes, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if ((st = check_dtype(kv_dtype))) return st;
  if (!Kc || !kmean || !codes || (K > 0 && !Wp) || U < 1 || cap < 1 || cap % 8) return MP_ERR_ARG;
  if (!all_a16(Kc, Wp, kmean, codes, ws)) return MP_ERR_ARG;
  if (U > 65535) return MP_ERR_UNSUPPORTED;
  if (n < 1 || n > cap) return MP_ERR_CAPACITY;
  if (!ws || ws_bytes < mp_build_ws_bytes(U, n, d)) return MP_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_kmean(Kc, kv_dtype, U, n, cap, (double *)ws, kmean_parts(n), kmean, s);
  if (e != hipSuccess) return MP_ERR_HIP;
  e = launch_encode(kv_dtype, Kc, cap * D, D, kmean, D, 0, U, n, Wp, K, L, codes, (int64_t)L * cap, 1, cap,
                    nullptr, 0, 0, nullptr, nullptr, s);
  return hip_status(e);
}

int mp_append(const void *k_new, const void *v_new, void *Kc, void *Vc, int kv_dtype, int64_t U, int64_t n,
              int64_t cap, int d, const float *kmean, const void *Wp, int K, int L, uint16_t *codes, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if ((st = check_dtype(kv_dtype))) return st;
  if (!k_new || !v_new || !Kc || !Vc || !kmean || !codes || (K > 0 && !Wp) || U < 1 || cap < 1 || cap % 8 ||
      n < 0)
    return MP_ERR_ARG;
  if (!all_a16(k_new, v_new, Kc, Vc, kmean, Wp, codes)) return MP_ERR_ARG;
  if (n >= cap) return MP_ERR_CAPACITY;
  const size_t es = kv_dtype == MP_BF16 ? 2 : 4;
  // one "unit" of U rows; row u has its own mean, cache row and code column
  hipError_t e = launch_encode(kv_dtype, k_new, 0, D, kmean, 0, D, 1, U, Wp, K, L, codes + n, 0, (int64_t)L * cap,
                               cap, (char *)Kc + (size_t)n * D * es, 0, cap * D, v_new,
                               (char *)Vc + (size_t)n * D * es, as_stream(stream));
  return hip_status(e);
}

size_t mp_proj_bytes_lift(int d, int K, int L) {
  const size_t base = mp_proj_bytes(d, K, L);
  if (base == 0 || K < 1) return 0;
  return base + (size_t)enc_ntiles(K, L) * 32 * sizeof(uint16_t);
}

int mp_proj_pack_lift(const float *W, int d, int K, int L, void *Wp, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if (K < 1) return MP_ERR_UNSUPPORTED;  // the lift needs projections
  if (!W || !Wp) return MP_ERR_ARG;
  if (!all_a16(Wp)) return MP_ERR_ARG;
  hipStream_t s = as_stream(stream);
  if (launch_proj_pack(W, K, L, Wp, s) != hipSuccess) return MP_ERR_HIP;
  return hip_status(launch_proj_pack_lift(W, K, L, (uint16_t *)((char *)Wp + mp_proj_bytes(d, K, L)), s));
}

int mp_build_codes_lift(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, int d, const void *Wp, int K,
                        int L, float *kmean, float *rlift, uint16_t *codes, void *ws, size_t ws_bytes, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if (K < 1) return MP_ERR_UNSUPPORTED;
  if ((st = check_dtype(kv_dtype))) return st;
  if (!Kc || !kmean || !rlift || !codes || !Wp || U < 1 || cap < 1 || cap % 8) return MP_ERR_ARG;
  if (!all_a16(Kc, Wp, kmean, codes, ws)) return MP_ERR_ARG;
  if (U > 65535) return MP_ERR_UNSUPPORTED;
  if (n < 1 || n > cap) return MP_ERR_CAPACITY;
  if (!ws || ws_bytes < mp_build_ws_bytes(U, n, d)) return MP_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  const int np = kmean_parts(n);
  if (launch_kmean(Kc, kv_dtype, U, n, cap, (double *)ws, np, kmean, s) != hipSuccess) return MP_ERR_HIP;
  if (launch_lift_radius(Kc, kv_dtype, U, n, cap, kmean, (double *)ws, np, rlift, s) != hipSuccess) return MP_ERR_HIP;
  EncJob j = make_job(Kc, cap * D, D, kmean, D, 0, U, n, codes, (int64_t)L * cap, 1, cap, nullptr, 0, 0, nullptr,
                      nullptr);
  j.rl = rlift;
  j.rl_su = 1;
  j.rl_si = 0;
  return hip_status(launch_encode_jobs(kv_dtype, &j, 1, Wp, K, L, s,
                                       (const uint16_t *)((const char *)Wp + mp_proj_bytes(d, K, L))));
}

int mp_append_lift(const void *k_new, const void *v_new, void *Kc, void *Vc, int kv_dtype, int64_t U, int64_t n,
                   int64_t cap, int d, const float *kmean, const float *rlift, const void *Wp, int K, int L,
                   uint16_t *codes, void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if (K < 1) return MP_ERR_UNSUPPORTED;
  if ((st = check_dtype(kv_dtype))) return st;
  if (!k_new || !v_new || !Kc || !Vc || !kmean || !rlift || !codes || !Wp || U < 1 || cap < 1 || cap % 8 || n < 0)
    return MP_ERR_ARG;
  if (!all_a16(k_new, v_new, Kc, Vc, kmean, Wp, codes)) return MP_ERR_ARG;
  if (n >= cap) return MP_ERR_CAPACITY;
  const size_t es = kv_dtype == MP_BF16 ? 2 : 4;
  EncJob j = make_job(k_new, 0, D, kmean, 0, D, 1, U, codes + n, 0, (int64_t)L * cap, cap,
                      (char *)Kc + (size_t)n * D * es, 0, cap * D, v_new, (char *)Vc + (size_t)n * D * es);
  j.rl = rlift;  // row i is unit i's new key
  j.rl_su = 0;
  j.rl_si = 1;
  return hip_status(launch_encode_jobs(kv_dtype, &j, 1, Wp, K, L, as_stream(stream),
                                       (const uint16_t *)((const char *)Wp + mp_proj_bytes(d, K, L))));
}

size_t mp_planes_bytes(int64_t U, int64_t cap, int K, int L) {
  if (U < 1 || cap < 1 || K < 1 || K > 16 || L < 2 || L > MAX_L || K * L > 4096) return 0;
  return (size_t)U * (size_t)((cap + SCAN_TILE - 1) / SCAN_TILE) * (size_t)K * (size_t)L * 16 * sizeof(uint32_t);
}

int mp_build_planes(const uint16_t *codes, int64_t U, int64_t n0, int64_t n1, int64_t cap, int K, int L,
                    uint32_t *planes, void *stream) {
  if (L < 2 || L > MAX_L || K > 16 || K * L > 4096) return MP_ERR_UNSUPPORTED;
  if (!codes || !planes || U < 1 || cap < 1 || cap % 8 || K < 1) return MP_ERR_ARG;
  if (!all_a16(codes, planes)) return MP_ERR_ARG;
  if (n0 < 0 || n0 > n1 || n1 > cap || n0 % SCAN_TILE || n1 % SCAN_TILE) return MP_ERR_ARG;
  const int64_t nt = (n1 - n0) / SCAN_TILE;
  if (U * nt * L >= ((int64_t)1 << 31)) return MP_ERR_UNSUPPORTED;  // one block per (unit, tile, table)
  return hip_status(launch_plane_build(codes, U, cap, K, L, n0 / SCAN_TILE, nt, planes, as_stream(stream)));
}

size_t mp_buckets_bytes(int64_t U, int64_t cap, int K, int L) {
  if (U < 1 || cap < 1 || K < 1 || K > MAX_BK_K || L < 2 || L > MAX_L || K * L > 4096) return 0;
  return bucket_layout(nullptr, U, cap, K, L).bytes;
}

int mp_build_buckets(const uint16_t *codes, int64_t U, int64_t n0, int64_t n1, int64_t cap, int K, int L,
                     void *buckets, size_t buckets_bytes, void *stream) {
  if (L < 2 || L > MAX_L || K < 1 || K > MAX_BK_K || K * L > 4096) return MP_ERR_UNSUPPORTED;
  if (!codes || !buckets || U < 1 || cap < 1 || cap % 8) return MP_ERR_ARG;
  if (!all_a16(codes, buckets)) return MP_ERR_ARG;
  if (n0 < 0 || n0 > n1 || n1 > cap || n0 % BK_R || n1 % SCAN_TILE) return MP_ERR_ARG;
  if (buckets_bytes < mp_buckets_bytes(U, cap, K, L)) return MP_ERR_WORKSPACE;
  const int64_t nc = (n1 + BK_R - 1) / BK_R - n0 / BK_R;
  if (U * L * nc >= ((int64_t)1 << 31)) return MP_ERR_UNSUPPORTED;  // one block per (unit, table, chunk)
  const BucketLayout bl = bucket_layout(buckets, U, cap, K, L);
  return hip_status(launch_bucket_build(codes, U, cap, K, L, n0, n1, bl, as_stream(stream)));
}

// Bucketed tables passed to a decode: whole 512-key tiles below n_buckets,
// used with threshold 2 (other thresholds scan the codes).
static int check_buckets(const void *buckets, int64_t n_buckets, int64_t n, int K) {
  if (!buckets) return MP_OK;
  if (!a16(buckets) || n_buckets < 0 || n_buckets > n || n_buckets % SCAN_TILE) return MP_ERR_ARG;
  if (K < 1 || K > MAX_BK_K) return MP_ERR_ARG;  // no bucketed table can exist for this K
  return MP_OK;
}

static int64_t list_keys(const void *buckets, int64_t n_buckets, int T) { return buckets && T == 2 ? n_buckets : 0; }

static int check_planes(const uint32_t *planes, int64_t n_planes, int64_t n) {
  if (!planes) return MP_OK;
  if (!a16(planes) || n_planes < 0 || n_planes > n || n_planes % SCAN_TILE) return MP_ERR_ARG;
  return MP_OK;
}

int mp_encode_queries(const void *q, int q_dtype, int64_t nq, int d, const void *Wp, int K, int L, uint16_t *qcodes,
                      void *stream) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if ((st = check_dtype(q_dtype))) return st;
  if (!q || !qcodes || (K > 0 && !Wp) || nq < 1) return MP_ERR_ARG;
  if (!all_a16(q, Wp)) return MP_ERR_ARG;
  hipError_t e = launch_encode(q_dtype, q, 0, D, nullptr, 0, 0, 1, nq, Wp, K, L, qcodes, 0, L, 1, nullptr, 0, 0,
                               nullptr, nullptr, as_stream(stream));
  return hip_status(e);
}

size_t mp_decode_ws_bytes(int B, int Hq, int Hkv, int64_t cap, int d, int L) {
  if (check_heads(B, Hq, Hkv) || d != D || cap < 1 || L < 2 || L > MAX_L) return 0;
  return decode_ws_layout(nullptr, B, Hq, Hkv, cap, L).bytes;
}

static int check_decode(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                        const float *kmean, int B, int Hq, int Hkv, int64_t n, int64_t cap, int d, int K, int L,
                        int T, int64_t nsh, int64_t nst, void *ws, size_t ws_bytes, bool caller_ws = true) {
  int st = check_shape(d, K, L);
  if (st) return st;
  if (T < 1 || T > L) return MP_ERR_UNSUPPORTED;
  if ((st = check_dtype(kv_dtype))) return st;
  if ((st = check_heads(B, Hq, Hkv))) return st;
  if (!q || !Kc || !Vc || !codes || !kmean || cap < 1 || cap % 8 || nsh < 0 || nst < 0) return MP_ERR_ARG;
  if (!all_a16(q, Kc, Vc, codes, kmean, ws)) return MP_ERR_ARG;
  if (n < 0 || n > cap) return MP_ERR_CAPACITY;
  // one sampling block per 512-key tile per unit, in a 1-D grid of < 2^31 threads
  if ((int64_t)B * Hkv * ((cap + SCAN_TILE - 1) / SCAN_TILE) > ((int64_t)1 << 23)) return MP_ERR_UNSUPPORTED;
  if (cap >= ((int64_t)1 << 26)) return MP_ERR_UNSUPPORTED;  // a scan batch's row offsets fit 32 bits
  if (caller_ws && (!ws || ws_bytes < mp_decode_ws_bytes(B, Hq, Hkv, cap, d, L))) return MP_ERR_WORKSPACE;
  return MP_OK;
}

// The sampling stage: the bucket lookup of the tiles below nl (when
// buckets are given), then the sampling kernel.
static int run_sample(int kv_dtype, const void *q, const void *Kc, const void *Vc, const uint16_t *codes,
                      const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap, int K,
                      int L, int T, int64_t nsh, int64_t nst, const DecodeGeom &geo, const DecodeWs &w, bool want_idx,
                      hipStream_t s, hipEvent_t ev0, hipEvent_t ev1, const uint32_t *planes, int64_t n_planes,
                      const void *buckets, int64_t nl, const float *rlift = nullptr) {
  if (nl > 0) {  // the events stay on the sampling kernel's own dispatch
    const BucketLayout bl = bucket_layout((void *)buckets, (int64_t)B * Hkv, cap, K, L);
    if (launch_bucket_lookup(qcodes, bl, B, Hq, Hkv, n, nl, cap, K, L, nsh, nst, geo, w, s) != hipSuccess)
      return MP_ERR_HIP;
  }
  return hip_status(launch_sample(kv_dtype, q, Kc, Vc, codes, kmean, qcodes, B, Hq, Hkv, n, cap, K, L, T, nsh, nst,
                                  geo, w, want_idx, s, ev0, ev1, planes, n_planes, nl, rlift));
}

int mp_decode_sample(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                     const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                     const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                     int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail, int want_idx, void *ws,
                     size_t ws_bytes, void *stream) {
  int st = check_decode(q, Kc, Vc, kv_dtype, codes, kmean, B, Hq, Hkv, n, cap, d, K, L, T, n_static_head,
                        n_static_tail, ws, ws_bytes);
  if (st) return st;
  if (!qcodes) return MP_ERR_ARG;
  if ((st = check_planes(planes, n_planes, n))) return st;
  if ((st = check_buckets(buckets, n_buckets, n, K))) return st;
  const DecodeGeom geo = decode_geom(B, Hkv, Hq, n, cap);
  const DecodeWs w = decode_ws_layout(ws, B, Hq, Hkv, cap, L);
  if (geo.nchunks == 0) return MP_OK;
  return run_sample(kv_dtype, q, Kc, Vc, codes, kmean, qcodes, B, Hq, Hkv, n, cap, K, L, T, n_static_head,
                    n_static_tail, geo, w, want_idx != 0, as_stream(stream), nullptr, nullptr, planes, n_planes,
                    buckets, list_keys(buckets, n_buckets, T));
}

int mp_decode_merge(int kv_dtype, int B, int Hq, int Hkv, int64_t n, int64_t cap, int d, int L, int T,
                    int64_t n_buckets, float *out, float *lse, int32_t *idx, int32_t *count, void *ws,
                    size_t ws_bytes, void *stream) {
  int st = check_heads(B, Hq, Hkv);
  if (st) return st;
  if ((st = check_dtype(kv_dtype))) return st;
  if (d != D || L < 2 || L > MAX_L || T < 1 || T > L) return MP_ERR_UNSUPPORTED;
  if (!out || cap < 1 || cap % 8) return MP_ERR_ARG;
  if (!all_a16(out, ws)) return MP_ERR_ARG;
  if (n < 0 || n > cap) return MP_ERR_CAPACITY;
  if (n_buckets < 0 || n_buckets > n || n_buckets % SCAN_TILE) return MP_ERR_ARG;
  if (!ws || ws_bytes < mp_decode_ws_bytes(B, Hq, Hkv, cap, d, L)) return MP_ERR_WORKSPACE;
  const DecodeGeom geo = decode_geom(B, Hkv, Hq, n, cap);
  const DecodeWs w = decode_ws_layout(ws, B, Hq, Hkv, cap, L);
  const int64_t nlt = (T == 2 ? n_buckets : 0) / SCAN_TILE;  // tiles the sampling stage took from bitmaps
  return hip_status(launch_merge(B, Hq, Hkv, n, L, geo, w, out, lse, idx, cap, count, as_stream(stream), nlt,
                                 sample_span(kv_dtype, Hq / Hkv, nlt, geo)));
}

static int decode_attn(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                       const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                       const float *kmean, const float *rlift, const void *Wp, int B, int Hq, int Hkv, int64_t n,
                       int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                       const uint16_t *qcodes_in, uint16_t *qcodes_out, float *out, float *lse, int32_t *idx,
                       int32_t *count, void *ws, size_t ws_bytes, void *stream) {
  int st = check_decode(q, Kc, Vc, kv_dtype, codes, kmean, B, Hq, Hkv, n, cap, d, K, L, T, n_static_head,
                        n_static_tail, ws, ws_bytes);
  if (st) return st;
  if (!out || (!qcodes_in && K > 0 && !Wp)) return MP_ERR_ARG;
  if (!all_a16(out, Wp)) return MP_ERR_ARG;
  if ((st = check_planes(planes, n_planes, n))) return st;
  if ((st = check_buckets(buckets, n_buckets, n, K))) return st;
  hipStream_t s = as_stream(stream);
  const DecodeGeom geo = decode_geom(B, Hkv, Hq, n, cap);
  const DecodeWs w = decode_ws_layout(ws, B, Hq, Hkv, cap, L);
  const uint16_t *qc = qcodes_in;
  if (!qc) {
    uint16_t *dst = qcodes_out ? qcodes_out : w.qcodes;
    hipError_t e = launch_encode(kv_dtype, q, 0, D, nullptr, 0, 0, 1, (int64_t)B * Hq, Wp, K, L, dst, 0, L, 1,
                                 nullptr, 0, 0, nullptr, nullptr, s);
    if (e != hipSuccess) return MP_ERR_HIP;
    qc = dst;
  }
  const int64_t nlt = list_keys(buckets, n_buckets, T) / SCAN_TILE;  // tiles with bitmaps
  if (geo.nchunks > 0) {
    st = run_sample(kv_dtype, q, Kc, Vc, codes, kmean, qc, B, Hq, Hkv, n, cap, K, L, T, n_static_head, n_static_tail,
                    geo, w, idx != nullptr, s, nullptr, nullptr, planes, n_planes, buckets,
                    list_keys(buckets, n_buckets, T), rlift);
    if (st) return st;
  }
  return hip_status(launch_merge(B, Hq, Hkv, n, L, geo, w, out, lse, idx, cap, count, s, nlt,
                                 sample_span(kv_dtype, Hq / Hkv, nlt, geo)));
}

int mp_decode_attn(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                   const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                   const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n, int64_t cap, int d, int K,
                   int L, int T, int64_t n_static_head, int64_t n_static_tail, const uint16_t *qcodes_in,
                   uint16_t *qcodes_out, float *out, float *lse, int32_t *idx, int32_t *count, void *ws,
                   size_t ws_bytes, void *stream) {
  return decode_attn(q, Kc, Vc, kv_dtype, codes, planes, n_planes, buckets, n_buckets, kmean, nullptr, Wp, B, Hq, Hkv,
                     n, cap, d, K, L, T, n_static_head, n_static_tail, qcodes_in, qcodes_out, out, lse, idx, count,
                     ws, ws_bytes, stream);
}

int mp_decode_attn_lift(const void *q, const void *Kc, const void *Vc, int kv_dtype, const uint16_t *codes,
                        const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                        const float *kmean, const float *rlift, const void *Wp, int B, int Hq, int Hkv, int64_t n,
                        int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                        const uint16_t *qcodes_in, uint16_t *qcodes_out, float *out, float *lse, int32_t *idx,
                        int32_t *count, void *ws, size_t ws_bytes, void *stream) {
  if (!rlift) return MP_ERR_ARG;
  return decode_attn(q, Kc, Vc, kv_dtype, codes, planes, n_planes, buckets, n_buckets, kmean, rlift, Wp, B, Hq, Hkv,
                     n, cap, d, K, L, T, n_static_head, n_static_tail, qcodes_in, qcodes_out, out, lse, idx, count,
                     ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------------------
// Static scratch of mp_decode_step_static: a fixed device array in the code
// object, one copy per GPU, used instead of a caller workspace.  Host code
// never passes `scratch` itself to a kernel or a copy (on the host the name
// only stands in for the symbol): it takes the array's device address once
// per device from hipGetSymbolAddress and uses that.
static __device__ __align__(256) unsigned char scratch[MP_STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<void *> scratch_ptr[MAX_DEVICES];
std::mutex scratch_mu;

// Device address of the current device's scratch (looked up on the first
// call on that device, with the device current).
int static_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MP_ERR_HIP;
  void *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MP_ERR_HIP;
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MP_OK;
}


// mp_decode_step: the public step entry points differ only in where the
// workspace comes from (the caller's ws, or with static_ws the library's
// static scratch, looked up once every argument has been validated).
int decode_step(const void *k_new, const void *v_new, const void *q, void *Kc, void *Vc, int kv_dtype,
                uint16_t *codes, const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                const float *kmean, const void *Wp, int B,
                int Hq, int Hkv, int64_t n, int64_t cap, int d, int K, int L, int T, int64_t n_static_head,
                int64_t n_static_tail, float *out, float *lse, int32_t *idx, int32_t *count, void *ws,
                size_t ws_bytes, void *sample_events, void *stream, bool static_ws) {
  const bool app = k_new != nullptr;
  if (app && !v_new) return MP_ERR_ARG;
  if (app && (n < 0 || n >= cap)) return MP_ERR_CAPACITY;
  const int64_t nd = app ? n + 1 : n;  // keys the decode sees
  int st = check_decode(q, Kc, Vc, kv_dtype, codes, kmean, B, Hq, Hkv, nd, cap, d, K, L, T, n_static_head,
                        n_static_tail, ws, ws_bytes, !static_ws);
  if (st) return st;
  if (!out || (K > 0 && !Wp)) return MP_ERR_ARG;
  if (!all_a16(out, Wp, k_new, v_new)) return MP_ERR_ARG;
  if ((st = check_planes(planes, n_planes, n))) return st;  // the keys before the append
  if ((st = check_buckets(buckets, n_buckets, n, K))) return st;
  if (static_ws) {
    if (mp_decode_ws_bytes(B, Hq, Hkv, cap, d, L) > (size_t)MP_STATIC_SCRATCH_BYTES) return MP_ERR_SCRATCH;
    if ((st = static_scratch(&ws))) return st;
  }
  hipStream_t s = as_stream(stream);
  const int64_t U = (int64_t)B * Hkv;
  const DecodeGeom geo = decode_geom(B, Hkv, Hq, nd, cap);
  const DecodeWs w = decode_ws_layout(ws, B, Hq, Hkv, cap, L);
  const size_t es = kv_dtype == MP_BF16 ? 2 : 4;
  // one launch: the appended keys (frozen means, codes at column n, raw rows
  // copied) and the queries (uncentred)
  EncJob jobs[2];
  int nj = 0;
  if (app)
    jobs[nj++] = make_job(k_new, 0, D, kmean, 0, D, 1, U, codes + n, 0, (int64_t)L * cap, cap,
                          (char *)Kc + (size_t)n * D * es, 0, cap * D, v_new, (char *)Vc + (size_t)n * D * es);
  jobs[nj++] = make_job(q, 0, D, nullptr, 0, 0, 1, (int64_t)B * Hq, w.qcodes, 0, L, 1, nullptr, 0, 0, nullptr,
                        nullptr);
  if (launch_encode_jobs(kv_dtype, jobs, nj, Wp, K, L, s) != hipSuccess) return MP_ERR_HIP;
  // the events ride on the sampling kernel's dispatch (its own start and end)
  hipEvent_t *ev = (hipEvent_t *)sample_events;
  if (geo.nchunks > 0) {
    st = run_sample(kv_dtype, q, Kc, Vc, codes, kmean, w.qcodes, B, Hq, Hkv, nd, cap, K, L, T, n_static_head,
                    n_static_tail, geo, w, idx != nullptr, s, ev ? ev[0] : nullptr, ev ? ev[1] : nullptr, planes,
                    n_planes, buckets, list_keys(buckets, n_buckets, T));
    if (st) return st;
  } else if (ev && (hipEventRecord(ev[0], s) != hipSuccess || hipEventRecord(ev[1], s) != hipSuccess)) {
    return MP_ERR_HIP;
  }
  const int64_t nlt = list_keys(buckets, n_buckets, T) / SCAN_TILE;  // tiles with bitmaps
  return hip_status(launch_merge(B, Hq, Hkv, nd, L, geo, w, out, lse, idx, cap, count, s, nlt,
                                 sample_span(kv_dtype, Hq / Hkv, nlt, geo)));
}

}  // namespace

extern "C" {

int mp_decode_step(const void *k_new, const void *v_new, const void *q, void *Kc, void *Vc, int kv_dtype,
                   uint16_t *codes, const uint32_t *planes, int64_t n_planes, const void *buckets, int64_t n_buckets,
                   const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                   int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail, float *out, float *lse,
                   int32_t *idx, int32_t *count, void *ws, size_t ws_bytes, void *sample_events, void *stream) {
  return decode_step(k_new, v_new, q, Kc, Vc, kv_dtype, codes, planes, n_planes, buckets, n_buckets, kmean, Wp, B,
                     Hq, Hkv, n, cap, d,
                     K, L, T, n_static_head, n_static_tail, out, lse, idx, count, ws, ws_bytes, sample_events,
                     stream, false);
}

int mp_decode_step_static(const void *k_new, const void *v_new, const void *q, void *Kc, void *Vc, int kv_dtype,
                          uint16_t *codes, const uint32_t *planes, int64_t n_planes, const void *buckets,
                          int64_t n_buckets, const float *kmean, const void *Wp, int B, int Hq, int Hkv, int64_t n,
                          int64_t cap, int d, int K, int L, int T, int64_t n_static_head, int64_t n_static_tail,
                          float *out, float *lse, int32_t *idx, int32_t *count, void *sample_events, void *stream) {
  return decode_step(k_new, v_new, q, Kc, Vc, kv_dtype, codes, planes, n_planes, buckets, n_buckets, kmean, Wp, B,
                     Hq, Hkv, n, cap, d,
                     K, L, T, n_static_head, n_static_tail, out, lse, idx, count, nullptr, 0, sample_events, stream,
                     true);
}

}  // extern "C"
