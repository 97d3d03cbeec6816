// Sampled decode attention of MagicPIG (arXiv 2410.16179v2, Section 4.3,
// Equations 9-11, Algorithm 1): collision scan over the table-major code
// store, compaction of the keys that collide in at least two tables, the
// importance weight exp(q.k/sqrt(d)) / P, split self-normalised attention and
// the log-sum-exp merge of the splits (Section 4.4 "On-device cache").
#include "mp_internal.h"

namespace mp {

constexpr uint32_t FORCED = 0x8000u;  // entry flag: forced key (probability 1)
constexpr int MAX_CHUNK_TILES = 4;
constexpr int MAX_CHUNK = MAX_CHUNK_TILES * SCAN_TILE;

DecodeGeom decode_geom(int B, int Hkv, int64_t n, int64_t cap) {
  DecodeGeom g;
  g.U = (int64_t)B * Hkv;
  const int64_t tiles = g.U * ((n + SCAN_TILE - 1) / SCAN_TILE);
  g.chunk_tiles = tiles < 2048 ? 1 : (tiles < 8192 ? 2 : 4);
  g.chunk = (int64_t)g.chunk_tiles * SCAN_TILE;
  g.nchunks = (n + g.chunk - 1) / g.chunk;
  g.nchunks_max = (cap + SCAN_TILE - 1) / SCAN_TILE;  // bound for any chunk size
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeWs decode_ws_layout(void *base, int B, int Hq, int Hkv, int64_t cap, int L) {
  const int64_t U = (int64_t)B * Hkv;
  const int G = Hq / Hkv;
  const int64_t ncm = (cap + SCAN_TILE - 1) / SCAN_TILE;
  const int64_t ent_per_unit = (cap + MAX_CHUNK - 1) / MAX_CHUNK * MAX_CHUNK;
  size_t off = 0;
  DecodeWs w;
  char *p = (char *)base;
  w.qcodes = (uint16_t *)(p + off);
  off = align256(off + sizeof(uint16_t) * (size_t)B * Hq * L);
  w.part = (float *)(p + off);
  off = align256(off + sizeof(float) * (size_t)U * ncm * G * PSTRIDE);
  w.ent = (uint32_t *)(p + off);
  off = align256(off + sizeof(uint32_t) * (size_t)U * ent_per_unit);
  w.ent_cnt = (int32_t *)(p + off);
  off = align256(off + sizeof(int32_t) * (size_t)U * ncm);
  w.bytes = off;
  return w;
}

// --------------------------------------------------------------------------
// ln P for a key at cosine `c` from the query (Equation 10):
//   u = 1 - acos(c)/pi = acos(-c)/pi,  p = u^K,
//   P = 1 - (1-p)^L - L p (1-p)^(L-1)   (at least two of L tables).
// The closed form cancels for small p, so for L p < 1 it is summed as the
// binomial tail from j = 2: ln P = ln C(L,2) + 2 ln p + (L-2) ln(1-p)
// + ln(1 + sum_{j>2} t_j/t_2) with t_{j+1}/t_j = (L-j)/(j+1) * p/(1-p);
// for L p >= 1 the closed form is evaluated as
// ln(-expm1((L-1) ln(1-p) + ln(1 + (L-1) p))).
__device__ inline float log_sampling_prob(float c, int K, int L) {
  if (K == 0) return 0.0f;  // p = 1: every table collides, P = 1
  c = fminf(1.0f, fmaxf(-1.0f, c));
  const float u = acosf(-c) * 0.318309886183790671538f;
  const float lnp = (float)K * logf(u);
  const float p = expf(lnp);
  const float Lf = (float)L;
  if (Lf * p < 1.0f) {
    const float r = p / (1.0f - p);
    float term = 1.0f, sum = 1.0f;
    for (int j = 2; j < L && j < 40; ++j) {
      term *= (float)(L - j) / (float)(j + 1) * r;
      sum += term;
      if (term < 1e-8f * sum) break;
    }
    return logf(0.5f * Lf * (Lf - 1.0f)) + 2.0f * lnp + (Lf - 2.0f) * log1pf(-p) + logf(sum);
  }
  return logf(-expm1f((Lf - 1.0f) * log1pf(-p) + log1pf((Lf - 1.0f) * p)));
}

// Sum over the 16 lanes of a DPP row (each lane ends with the row sum).
__device__ inline float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

template <typename T>
__device__ inline void ld8(const T *p, float (&v)[8]);
template <>
__device__ inline void ld8<float>(const float *p, float (&v)[8]) {
  const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
}
template <>
__device__ inline void ld8<__bf16>(const __bf16 *p, float (&v)[8]) {
  const bf16x8 a = *(const bf16x8 *)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}

// Raw 8-element row slices kept in registers between the gather and its use.
template <typename T>
struct Raw8;
template <>
struct Raw8<__bf16> {
  uint4 a;
  __device__ void load(const __bf16 *p) { a = *(const uint4 *)p; }
  __device__ void get(float (&v)[8]) const {
    const bf16x8 b = __builtin_bit_cast(bf16x8, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)b[e];
  }
};
template <>
struct Raw8<float> {
  uint4 a, b;
  __device__ void load(const float *p) { a = *(const uint4 *)p; b = *(const uint4 *)(p + 4); }
  __device__ void get(float (&v)[8]) const {
    const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = x[e]; v[e + 4] = y[e]; }
  }
};

// --------------------------------------------------------------------------
// One block = one chunk (chunk_tiles x 512 keys) of one unit (batch, KV head)
// for all G query heads of that KV head.
//
// Scan: per 512-key tile, lane l of wave w reads 16 bytes (8 keys) of the
// codes of tables w, w+4, w+8, ... and counts, for every head, the tables
// whose code differs from the query's (xor, packed min with 1, packed add:
// two keys per 32-bit word).  The four waves' counts are added through LDS;
// key i is sampled for head h when L - mismatches >= 2.  Forced keys (the
// static head/tail ranges) are sampled for every head with P = 1.
//
// Compaction: wave ballots + popcounts give each key's rank, so the chunk's
// union list (key, head mask) is built in LDS in ascending key order.
//
// Attention: 16-lane groups take list entries round robin; a group gathers
// the key and value rows (16 lanes x 8 elements), reduces q_h.k and |k-mu|^2
// across its row, lane h of the group turns head h's numbers into the
// log-weight s - ln P, and every head with its mask bit set folds the value
// row into an online softmax (m, l, o).  The 16 groups are then merged by
// log-sum-exp and one partial record per head is written.
template <typename T, int GM>
__global__ __launch_bounds__(256, 2) void sample_kernel(
    const T *__restrict__ q, const T *__restrict__ Kc, const T *__restrict__ Vc, const uint16_t *__restrict__ codes,
    const float *__restrict__ kmean, const uint16_t *__restrict__ qcodes, int Hq, int Hkv, int G, int64_t n,
    int64_t cap, int K, int L, int64_t nsh, int64_t nst, int chunk_tiles, int64_t nchunks, float scale,
    uint32_t one2, float *__restrict__ part, uint32_t *__restrict__ ent, int32_t *__restrict__ ent_cnt) {
  __shared__ uint32_t qpk[MAX_L * GM];
  __shared__ uint4 red[4][GM][64];
  __shared__ uint16_t ukey[MAX_CHUNK];
  __shared__ uint16_t umask[MAX_CHUNK];
  __shared__ int wtot[4];
  __shared__ int hcnt[GM];
  __shared__ int nu_sh;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t u = blockIdx.y;
  const int64_t c = blockIdx.x;
  const int64_t b = u / Hkv, kvh = u % Hkv;
  const int64_t qrow0 = b * Hq + kvh * G;  // first query head of this unit
  const int64_t chunk = (int64_t)chunk_tiles * SCAN_TILE;
  const int64_t cbase = c * chunk;
  const uint16_t headbits = (uint16_t)((1u << G) - 1u);

  for (int i = tid; i < L * GM; i += 256) {
    const int l = i / GM, h = i % GM;
    const uint32_t code = h < G ? qcodes[(qrow0 + h) * L + l] : 0u;
    qpk[i] = code | (code << 16);
  }
  if (tid < GM) hcnt[tid] = 0;
  if (tid == 0) nu_sh = 0;
  __syncthreads();

  const u16x2 one = __builtin_bit_cast(u16x2, one2);
  const uint16_t *ucodes = codes + u * (int64_t)L * cap;

  // ------------------------------------------------------------ scan + compaction
  for (int tt = 0; tt < chunk_tiles; ++tt) {
    const int64_t tbase = cbase + (int64_t)tt * SCAN_TILE;
    if (tbase >= n) break;
    const int64_t key0 = tbase + 8 * lane;
    const bool lane_ok = key0 < n;
    uint32_t acc[GM][4];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[h][w] = 0;

    const int ntw = (L - wave + 3) / 4;  // tables of this wave: wave, wave+4, ...
    for (int j0 = 0; j0 < ntw; j0 += 8) {
      uint4 cw[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int l = wave + 4 * (j0 + jj);
        cw[jj] = make_uint4(0, 0, 0, 0);
        if (j0 + jj < ntw && lane_ok) cw[jj] = *(const uint4 *)(ucodes + (int64_t)l * cap + key0);
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        if (j0 + jj < ntw) {
          const int l = wave + 4 * (j0 + jj);
          const uint32_t w4[4] = {cw[jj].x, cw[jj].y, cw[jj].z, cw[jj].w};
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            const uint32_t Q = qpk[l * GM + h];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const u16x2 x = __builtin_bit_cast(u16x2, w4[w] ^ Q);
              acc[h][w] += __builtin_bit_cast(uint32_t, __builtin_elementwise_min(x, one));
            }
          }
        }
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) red[wave][h][lane] = make_uint4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
    __syncthreads();

    // thread tid owns tile keys 2*tid and 2*tid+1: lane tid/4, word tid%4
    const int64_t klo = tbase + 2 * tid;
    uint32_t mlo = 0, mhi = 0;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        uint32_t s = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) s += ((const uint32_t *)&red[w][h][tid >> 2])[tid & 3];
        const int mis_lo = (int)(s & 0xffffu), mis_hi = (int)(s >> 16);
        mlo |= (uint32_t)(L - mis_lo >= 2) << h;
        mhi |= (uint32_t)(L - mis_hi >= 2) << h;
      }
    }
    if (klo < nsh || klo >= n - nst) mlo = headbits | FORCED;
    if (klo + 1 < nsh || klo + 1 >= n - nst) mhi = headbits | FORCED;
    if (klo >= n) mlo = 0;
    if (klo + 1 >= n) mhi = 0;

    const bool flo = (mlo & headbits) != 0, fhi = (mhi & headbits) != 0;
    const uint64_t blo = __ballot(flo), bhi = __ballot(fhi);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int pre = __popcll(blo & lt) + __popcll(bhi & lt);
    if (lane == 0) wtot[wave] = __popcll(blo) + __popcll(bhi);
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const int ch = __popcll(__ballot((mlo >> h) & 1)) + __popcll(__ballot((mhi >> h) & 1));
        if (lane == 0 && ch) atomicAdd(&hcnt[h], ch);
      }
    }
    __syncthreads();
    int off = nu_sh;
    for (int w = 0; w < wave; ++w) off += wtot[w];
    const int64_t kl_local = klo - cbase;
    if (flo) {
      ukey[off + pre] = (uint16_t)kl_local;
      umask[off + pre] = (uint16_t)mlo;
      if (ent) ent[(u * nchunks + c) * chunk + off + pre] = (uint32_t)kl_local | ((mlo & headbits) << 16);
    }
    if (fhi) {
      const int p2 = off + pre + (flo ? 1 : 0);
      ukey[p2] = (uint16_t)(kl_local + 1);
      umask[p2] = (uint16_t)mhi;
      if (ent) ent[(u * nchunks + c) * chunk + p2] = (uint32_t)(kl_local + 1) | ((mhi & headbits) << 16);
    }
    __syncthreads();
    if (tid == 0) nu_sh += wtot[0] + wtot[1] + wtot[2] + wtot[3];
    __syncthreads();
  }
  const int nu = nu_sh;
  if (ent_cnt && tid == 0) ent_cnt[u * nchunks + c] = nu;

  // ------------------------------------------------------------ weighting + attention
  const int j16 = lane & 15, grp = tid >> 4;
  float qf[GM][8], mv[8];
  {
    ld8<float>(kmean + u * D + 8 * j16, mv);
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) ld8<T>(q + (qrow0 + h) * D + 8 * j16, qf[h]);
      else
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] = 0.0f;
    }
  }
  float qn_mine = 1.0f, qmu_mine = 0.0f;  // |q_h| and q_h.mu of head h = j16
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    float a = 0.0f, bq = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { a += qf[h][e] * qf[h][e]; bq += qf[h][e] * mv[e]; }
    a = row16_sum(a);
    bq = row16_sum(bq);
    if (j16 == h) { qn_mine = sqrtf(a); qmu_mine = bq; }
  }

  float m[GM], lsum[GM], o[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    lsum[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.0f;
  }

  const T *Ku = Kc + u * cap * D + 8 * j16;
  const T *Vu = Vc + u * cap * D + 8 * j16;
  Raw8<T> kr, vr;
  int e = grp;
  if (e < nu) {
    const int64_t key = cbase + ukey[e];
    kr.load(Ku + key * D);
    vr.load(Vu + key * D);
  }
  for (; e < nu; e += 16) {
    const uint32_t mk = umask[e];
    float kv[8], vv[8];
    kr.get(kv);
    vr.get(vv);
    if (e + 16 < nu) {  // prefetch the group's next entry
      const int64_t key = cbase + ukey[e + 16];
      kr.load(Ku + key * D);
      vr.load(Vu + key * D);
    }
    float nc2 = 0.0f, dk[GM];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float ct = kv[t] - mv[t];
      nc2 += ct * ct;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) a += qf[h][t] * kv[t];
      dk[h] = row16_sum(a);
    }
    nc2 = row16_sum(nc2);
    // lane h of the group computes head h's log-weight
    float my_dk = dk[0];
#pragma unroll
    for (int h = 1; h < GM; ++h)
      if (j16 == h) my_dk = dk[h];
    float lw = -INFINITY;
    if (j16 < G && ((mk >> j16) & 1u)) {
      float lnP = 0.0f;
      if (!(mk & FORCED)) {
        const float den = qn_mine * sqrtf(nc2);
        const float cosv = den > 0.0f ? (my_dk - qmu_mine) / den : 0.0f;
        lnP = log_sampling_prob(cosv, K, L);
      }
      lw = my_dk * scale - lnP;
    }
    const int gbase = lane & ~15;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h < G) {
        const float s = __shfl(lw, gbase + h);
        if (s > -INFINITY) {
          const float mn = fmaxf(m[h], s);
          const float alpha = __expf(m[h] - mn);  // 0 when m = -inf
          const float beta = __expf(s - mn);
          lsum[h] = lsum[h] * alpha + beta;
#pragma unroll
          for (int t = 0; t < 8; ++t) o[h][t] = o[h][t] * alpha + beta * vv[t];
          m[h] = mn;
        }
      }
    }
  }

  // merge the 4 groups of each wave (lanes xor 16, xor 32)
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
#pragma unroll
      for (int sh = 16; sh <= 32; sh <<= 1) {
        const float m2 = __shfl_xor(m[h], sh);
        const float l2 = __shfl_xor(lsum[h], sh);
        const float mn = fmaxf(m[h], m2);
        const float a = m[h] > -INFINITY ? __expf(m[h] - mn) : 0.0f;
        const float bb = m2 > -INFINITY ? __expf(m2 - mn) : 0.0f;
        lsum[h] = lsum[h] * a + l2 * bb;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float o2 = __shfl_xor(o[h][t], sh);
          o[h][t] = o[h][t] * a + o2 * bb;
        }
        m[h] = mn;
      }
    }
  }
  __syncthreads();  // red is reused below
  float *wst = (float *)&red[0][0][0];  // [4 waves][GM][130]: m, l, o[128]
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G && lane < 16) {
      float *r = wst + (wave * GM + h) * 130;
      if (lane == 0) { r[0] = m[h]; r[1] = lsum[h]; }
#pragma unroll
      for (int t = 0; t < 8; ++t) r[2 + 8 * lane + t] = o[h][t];
    }
  }
  __syncthreads();
  float *pout = part + (u * nchunks + c) * G * PSTRIDE;
  for (int i = tid; i < G * D; i += 256) {
    const int h = i / D, t = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wst[(w * GM + h) * 130]);
    float ls = 0.0f, os = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = wst[(w * GM + h) * 130];
      const float sc = mw > -INFINITY ? __expf(mw - M) : 0.0f;
      ls += wst[(w * GM + h) * 130 + 1] * sc;
      os += wst[(w * GM + h) * 130 + 2 + t] * sc;
    }
    float *rec = pout + h * PSTRIDE;
    rec[4 + t] = os;
    if (t == 0) {
      rec[0] = M;
      rec[1] = ls;
      rec[2] = __builtin_bit_cast(float, hcnt[h]);
      rec[3] = 0.0f;
    }
  }
}

hipError_t launch_sample(int dtype, const void *q, const void *Kc, const void *Vc, const uint16_t *codes,
                         const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                         int K, int L, int64_t nsh, int64_t nst, const DecodeGeom &geo, const DecodeWs &ws,
                         bool want_idx, hipStream_t s) {
  const int G = Hq / Hkv;
  const dim3 grid((unsigned)geo.nchunks, (unsigned)geo.U);
  const float scale = 1.0f / sqrtf((float)D);
  const uint32_t one2 = 0x00010001u;
  uint32_t *ent = want_idx ? ws.ent : nullptr;
  int32_t *ent_cnt = want_idx ? ws.ent_cnt : nullptr;
#define MP_SAMPLE(T, GMV)                                                                                        \
  sample_kernel<T, GMV><<<grid, 256, 0, s>>>((const T *)q, (const T *)Kc, (const T *)Vc, codes, kmean, qcodes,  \
                                             Hq, Hkv, G, n, cap, K, L, nsh, nst, geo.chunk_tiles, geo.nchunks,  \
                                             scale, one2, ws.part, ent, ent_cnt)
#define MP_SAMPLE_G(T) \
  do {                 \
    if (G == 1)        \
      MP_SAMPLE(T, 1); \
    else if (G == 2)   \
      MP_SAMPLE(T, 2); \
    else if (G <= 4)   \
      MP_SAMPLE(T, 4); \
    else               \
      MP_SAMPLE(T, 8); \
  } while (0)
  if (dtype == 0)
    MP_SAMPLE_G(__bf16);
  else
    MP_SAMPLE_G(float);
#undef MP_SAMPLE_G
#undef MP_SAMPLE
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Log-sum-exp merge of the per-chunk partials of one query head (one block
// of 128 threads, one output dimension each), and, when idx is requested,
// the ascending sampled-index list assembled from the chunks' union entries.
__global__ __launch_bounds__(128) void merge_kernel(const float *__restrict__ part, int Hq, int Hkv, int G,
                                                    int64_t nchunks, int64_t chunk, float *__restrict__ out,
                                                    float *__restrict__ lse, int32_t *__restrict__ count,
                                                    int32_t *__restrict__ idx, int64_t cap,
                                                    const uint32_t *__restrict__ ent,
                                                    const int32_t *__restrict__ ent_cnt) {
  __shared__ int wsum[2];
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / Hq, h = bh % Hq;
  const int64_t u = b * Hkv + h / G;
  const int hg = (int)(h % G);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float *p0 = part + (u * nchunks * G + hg) * PSTRIDE;
  const int64_t cs = (int64_t)G * PSTRIDE;
  float M = -INFINITY;
  for (int64_t ci = 0; ci < nchunks; ++ci) M = fmaxf(M, p0[ci * cs]);
  float l = 0.0f, acc = 0.0f;
  int cnt = 0;
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    const float *r = p0 + ci * cs;
    cnt += __builtin_bit_cast(int, r[2]);
    if (r[0] > -INFINITY) {
      const float sc = __expf(r[0] - M);
      l += r[1] * sc;
      acc += r[4 + t] * sc;
    }
  }
  out[bh * D + t] = l > 0.0f ? acc / l : 0.0f;
  if (t == 0) {
    if (lse) lse[bh] = l > 0.0f ? M + logf(l) : -INFINITY;
    if (count) count[bh] = cnt;
  }
  if (!idx) return;
  int32_t *dst = idx + bh * cap;
  int base = 0;
  for (int64_t ci = 0; ci < nchunks; ++ci) {
    // clamp: stays inside the workspace even if the entries were not written
    const int ne = min(max(ent_cnt[u * nchunks + ci], 0), (int)chunk);
    const uint32_t *src = ent + (u * nchunks + ci) * chunk;
    for (int e0 = 0; e0 < ne; e0 += 128) {
      const int e = e0 + t;
      uint32_t v = 0;
      bool f = false;
      if (e < ne) {
        v = src[e];
        f = (v >> (16 + hg)) & 1u;
      }
      const uint64_t bal = __ballot(f);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int pre = __popcll(bal & lt);
      if (lane == 0) wsum[wave] = __popcll(bal);
      __syncthreads();
      const int off = base + (wave ? wsum[0] : 0);
      if (f && off + pre < cap) dst[off + pre] = (int32_t)(ci * chunk + (v & 0xffffu));
      base += wsum[0] + wsum[1];
      __syncthreads();
    }
  }
}

hipError_t launch_merge(int B, int Hq, int Hkv, int64_t n, int L, const DecodeGeom &geo, const DecodeWs &ws,
                        float *out, float *lse, int32_t *idx, int64_t cap, int32_t *count, hipStream_t s) {
  (void)n;
  (void)L;
  const int G = Hq / Hkv;
  merge_kernel<<<dim3((unsigned)((int64_t)B * Hq)), 128, 0, s>>>(ws.part, Hq, Hkv, G, geo.nchunks, geo.chunk, out,
                                                                 lse, count, idx, cap, ws.ent, ws.ent_cnt);
  return hipGetLastError();
}

}  // namespace mp
