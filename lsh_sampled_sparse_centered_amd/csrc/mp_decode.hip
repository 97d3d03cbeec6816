// Sampled decode attention of MagicPIG (arXiv 2410.16179v2, Section 4.3,
// Equations 9-11, Algorithm 1): collision scan over the table-major code
// store, compaction of the keys that collide in at least two tables, the
// importance weight exp(q.k/sqrt(d)) / P, split self-normalised attention and
// the log-sum-exp merge of the splits (Section 4.4 "On-device cache").
#include <hip/hip_ext.h>

#include <cmath>

#include <type_traits>

#include "mp_internal.h"

namespace mp {

#ifndef MP_OCC
#define MP_OCC 7  // waves per SIMD the G <= 4 bf16 kernels are compiled for (72 VGPRs: one round at 96K)
#endif
#ifndef MP_OCC_F32
#define MP_OCC_F32 6  // fp32 caches (more registers per gathered row)
#endif
#ifndef MP_OCC8
#define MP_OCC8 5  // waves per SIMD the G = 8 kernels are compiled for (96 VGPRs)
#endif
#ifndef MP_SB
#define MP_SB 8  // code-store rows per load batch of a wave
#endif

constexpr uint32_t FORCED = 0x8000u;  // entry flag: forced key (probability 1)
constexpr int ATT_E = 32;  // list entries per attention round
constexpr int VT_STRIDE = 40;  // entries per row of the transposed value rows (32 + padding, 16-byte rows)

LnPCoef lnp_coef(int K, int L, int T) {
  LnPCoef c{};
  c.T = T;
  c.Kf = (float)K;
  c.Lf = (float)L;
  c.Lm1 = (float)(L - 1);
  c.Lm2 = (float)(L - 2);
  c.Tf = (float)T;
  c.LmT = (float)(L - T);
  c.lnct = (float)(std::lgamma((double)L + 1.0) - std::lgamma((double)T + 1.0) - std::lgamma((double)(L - T) + 1.0));
  double a = 1.0;  // C(L, 2+i) / C(L, 2), by the ratio C(L, k+1) / C(L, k) = (L-k)/(k+1)
  for (int i = 0; i < LNP_TERMS; ++i) {
    c.a[i] = (float)a;
    const int k = 2 + i;
    a = k < L ? a * (double)(L - k) / (double)(k + 1) : 0.0;
  }
  c.lnc2 = (float)std::log(0.5 * (double)L * (double)(L - 1));
  return c;
}

// One 512-key tile per block.
DecodeGeom decode_geom(int B, int Hkv, int Hq, int64_t n, int64_t cap) {
  (void)Hq;
  DecodeGeom g;
  g.U = (int64_t)B * Hkv;
  g.chunk = SCAN_TILE;
  g.nchunks = (n + SCAN_TILE - 1) / SCAN_TILE;
  g.nchunks_max = (cap + SCAN_TILE - 1) / SCAN_TILE;
  return g;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeWs decode_ws_layout(void *base, int B, int Hq, int Hkv, int64_t cap, int L) {
  const int64_t U = (int64_t)B * Hkv;
  const int G = Hq / Hkv;
  const int64_t ncm = (cap + SCAN_TILE - 1) / SCAN_TILE;
  const int64_t ent_per_unit = 2 * ncm * SCAN_TILE;  // up to 1024 entries per block
  // offsets first; pointers only into a real buffer (a NULL base asks for the size)
  size_t off = 0;
  DecodeWs w;
  auto at = [base](size_t o) -> void * { return base ? (char *)base + o : nullptr; };
  w.qcodes = (uint16_t *)at(off);
  off = align256(off + sizeof(uint16_t) * (size_t)B * Hq * L);
  w.part = (float *)at(off);
  off = align256(off + sizeof(float) * (size_t)U * ncm * G * PSTRIDE);
  w.ent = (uint32_t *)at(off);
  off = align256(off + sizeof(uint32_t) * (size_t)U * ent_per_unit);
  w.ent_cnt = (int32_t *)at(off);
  off = align256(off + sizeof(int32_t) * (size_t)U * ncm);
  w.bits = (uint32_t *)at(off);
  off = align256(off + sizeof(uint32_t) * (size_t)U * G * ncm * (SCAN_TILE / 32));
  w.bytes = off;
  return w;
}

// --------------------------------------------------------------------------
// ln P for a key at cosine `c` from the query (Equation 10):
//   u = 1 - acos(c)/pi = acos(-c)/pi,  p = u^K,
//   P = 1 - (1-p)^L - L p (1-p)^(L-1)   (at least two of L tables).
// The closed form cancels for small p, so for L p < 1 it is summed as the
// binomial tail from j = 2:
//   P = C(L,2) p^2 (1-p)^(L-2) * sum_i a_i r^i,  r = p/(1-p),
//   a_i = C(L, 2+i) / C(L, 2),
// with the a_i (i < LNP_TERMS) and ln C(L,2) computed on the host per L;
// with L p < 1 the terms from i = 12 on are below 3e-11 of the sum.  For
// L p >= 1 the closed form is evaluated as
// ln(-expm1((L-1) ln(1-p) + ln(1 + (L-1) p))).
// Any other threshold T (at least T of L tables): with r = p/(1-p),
//   L p <= T: P = C(L,T) p^T (1-p)^(L-T) * sum_{j>=T} t_j / t_T, where
//             t_{j+1}/t_j = (L-j)/(j+1) r; past the mode (<= T) the terms
//             only fall, and the sum stops once a term is below 1e-8 of it;
//   L p >  T: P = 1 - sum_{j<T} C(L,j) p^j (1-p)^(L-j) (P is not small there).
__device__ inline float log_sampling_prob_t(float lnp, float p, int L, int T, const LnPCoef &cf) {
  if (p >= 1.0f) return 0.0f;
  const float l1p = log1pf(-p), r = p / (1.0f - p);
  if (cf.Lf * p <= cf.Tf) {
    float sum = 1.0f, term = 1.0f;
    for (int j = T; j < L; ++j) {
      term *= (float)(L - j) * __builtin_amdgcn_rcpf((float)(j + 1)) * r;
      sum += term;
      if (term < 1e-8f * sum) break;
    }
    return cf.lnct + cf.Tf * lnp + cf.LmT * l1p + __logf(sum);
  }
  float term = __expf(cf.Lf * l1p), below = term;  // j = 0
  for (int j = 0; j + 1 < T; ++j) {
    term *= (float)(L - j) * __builtin_amdgcn_rcpf((float)(j + 1)) * r;
    below += term;
  }
  return log1pf(-fminf(below, 1.0f));
}

// acos(x) / pi for x in [-1, 1]: acos(|x|) = sqrt(1 - |x|) * a(|x|) with the
// degree-7 polynomial a of Abramowitz and Stegun, Handbook of Mathematical
// Functions, 4.4.46 (absolute error <= 2e-8 on [0, 1]), and
// acos(x) = pi - acos(-x) for x < 0.
__device__ inline float acos_over_pi(float x) {
  const float ax = fabsf(x);
  float a = -0.0012624911f;
  a = fmaf(a, ax, 0.0066700901f);
  a = fmaf(a, ax, -0.0170881256f);
  a = fmaf(a, ax, 0.0308918810f);
  a = fmaf(a, ax, -0.0501743046f);
  a = fmaf(a, ax, 0.0889789874f);
  a = fmaf(a, ax, -0.2145988016f);
  a = fmaf(a, ax, 1.5707963050f);
  const float t = __builtin_amdgcn_sqrtf(1.0f - ax) * a * 0.318309886183790671538f;
  return x < 0.0f ? 1.0f - t : t;
}
// The hardware's base-2 logarithm and exponential (one instruction each,
// about 1 ulp; no denormal scaling: their arguments here are normal or 0).
__device__ inline float hw_ln(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }
__device__ inline float hw_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.442695040888963407f); }
// ln(1 + x), x > -1, from the hardware logarithm with the rounding of 1 + x
// compensated: w = fl(1 + x), ln(1 + x) = ln(w) * x / (w - 1) (Goldberg,
// "What every computer scientist should know about floating-point
// arithmetic", Theorem 4).
__device__ inline float log1p_hw(float x) {
  const float w = 1.0f + x, d = w - 1.0f;
  return d == 0.0f ? x : hw_ln(w) * (x * __builtin_amdgcn_rcpf(d));
}
// The threshold-2 form above with hardware logarithms and exponentials and
// no divergent branch (both forms are evaluated and one is selected): all
// lanes of a wave take the same ~60 instructions.
__device__ inline float log_sampling_prob(float c, int K, int L, const LnPCoef &cf) {
  if (K == 0) return 0.0f;  // p = 1: every table collides, P = 1
  c = fminf(1.0f, fmaxf(-1.0f, c));
  const float u = acos_over_pi(-c);
  const float lnp = cf.Kf * hw_ln(u);
  const float p = hw_exp(lnp);
  if (cf.T != 2) return log_sampling_prob_t(lnp, p, L, cf.T, cf);
  const float l1p = log1p_hw(-p);  // ln(1 - p)
  // L p < 1: the binomial tail from j = 2 (no cancellation for small p)
  const float r = p * __builtin_amdgcn_rcpf(1.0f - p);
  float sum = cf.a[LNP_TERMS - 1];
#pragma unroll
  for (int i = LNP_TERMS - 2; i >= 0; --i) sum = fmaf(sum, r, cf.a[i]);
  const float small = cf.lnc2 + 2.0f * lnp + cf.Lm2 * l1p + hw_ln(sum);
  // L p >= 1: ln(1 - e^y), y = (L-1) ln(1-p) + ln(1 + (L-1) p); there
  // e^y <= 0.74, so 1 - e^y keeps its precision
  const float y = cf.Lm1 * l1p + hw_ln(fmaf(cf.Lm1, p, 1.0f));
  const float large = hw_ln(1.0f - hw_exp(y));
  return cf.Lf * p < 1.0f ? small : large;
}

// Lane exchanges within a DPP row of 16 lanes (quad_perm [1,0,3,2] and
// [2,3,0,1], row_half_mirror, row_mirror: after the four steps every lane of
// the row has combined all 16) and a lane-xor swizzle across rows.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int XM>
__device__ inline float swz_xor(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (XM << 10) | 0x1f));
}
// Sum / maximum over the 16 lanes of a DPP row (each lane ends with the row's).
__device__ inline float row16_sum(float x) {
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  x += dpp_mov<0x141>(x);
  return x + dpp_mov<0x140>(x);
}
__device__ inline float row16_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x141>(x));
  return fmaxf(x, dpp_mov<0x140>(x));
}
// Maximum and sum over each half (32 lanes) of the wave, every lane ending
// with its half's result: the row's, then one swizzle between the two rows.
__device__ inline float xor32_max(float x) {
  x = row16_max(x);
  return fmaxf(x, swz_xor<16>(x));
}
__device__ inline float xor32_sum(float x) {
  x = row16_sum(x);
  return x + swz_xor<16>(x);
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
  __device__ void zero() { a = uint4{0u, 0u, 0u, 0u}; }
  __device__ void get(float (&v)[8]) const {
    const bf16x8 b = __builtin_bit_cast(bf16x8, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (float)b[e];
  }
  __device__ void store(__bf16 *p) const { *(uint4 *)p = a; }
};
template <>
struct Raw8<float> {
  uint4 a, b;
  __device__ void load(const float *p) { a = *(const uint4 *)p; b = *(const uint4 *)(p + 4); }
  __device__ void zero() { a = b = uint4{0u, 0u, 0u, 0u}; }
  __device__ void get(float (&v)[8]) const {
    const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) { v[e] = x[e]; v[e + 4] = y[e]; }
  }
  __device__ void store(float *p) const {
    *(uint4 *)p = a;
    *(uint4 *)(p + 4) = b;
  }
};

// N consecutive elements of a staged LDS row, as floats.
template <typename T, int N>
__device__ inline void ldv(const T *p, float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = (float)p[i];
}

// Two list entries in a 16-lane group (lane j16 holds elements 8*j16 .. +7
// of each row): stage both value row slices in LDS, reduce |k - mu|^2 and
// q_h.k over the rows (every lane ends with every sum), then lane j16 forms
// the log-weight s - ln P of entry (j16 < 8 ? e0 : e1) for head j16 % 8, or
// -inf when that head did not sample the key.  q, mu, |q_h| and q_h.mu come
// from LDS.  The second entry is ignored when !ok1.
template <typename T, int GM>
__device__ inline void entry_pair(const Raw8<T> &k0, const Raw8<T> &v0, const Raw8<T> &k1, const Raw8<T> &v1,
                                  bool ok1, int e0, int e1, uint32_t mk0, uint32_t mk1, int j16, int G, int K, int L,
                                  const LnPCoef &cf, float scale, const T (*qsh)[D], const float *msh,
                                  const f32x4 *hst, T (*vrows)[D], float (*lw)[ATT_E], float rl) {
  float kv0[8], kv1[8], mv[8];
  k0.get(kv0);
  k1.get(kv1);
  v0.store(vrows[e0] + 8 * j16);
  if (ok1) v1.store(vrows[e1] + 8 * j16);
  ld8<float>(msh + 8 * j16, mv);
  float n0 = 0.0f, n1 = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float c0 = kv0[t] - mv[t], c1 = kv1[t] - mv[t];
    n0 += c0 * c0;
    n1 += c1 * c1;
  }
  n0 = row16_sum(n0);
  n1 = row16_sum(n1);
  const int hh = j16 & 7;
  const bool second = j16 >= 8;
  float dk = 0.0f;
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h < G) {
      float qv[8];
      ld8<T>(&qsh[h][8 * j16], qv);
      float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        a0 += qv[t] * kv0[t];
        a1 += qv[t] * kv1[t];
      }
      a0 = row16_sum(a0);
      a1 = row16_sum(a1);
      if (hh == h) dk = second ? a1 : a0;
    }
  }
  if (hh < G && (!second || ok1)) {
    const uint32_t mk = second ? mk1 : mk0;
    float w = -INFINITY;
    if ((mk >> hh) & 1u) {
      float lnP = 0.0f;
      if (!(mk & FORCED)) {
        const f32x4 hs = hst[hh];
        const float den = hs[0] * (rl > 0.0f ? rl : __builtin_amdgcn_sqrtf(second ? n1 : n0));
        const float cosv = den > 0.0f ? (dk - hs[1]) * __builtin_amdgcn_rcpf(den) : 0.0f;
        lnP = log_sampling_prob(cosv, K, L, cf);
      }
      w = dk * scale - lnP;
    }
    lw[hh][second ? e1 : e0] = w;
  }
}

// --------------------------------------------------------------------------
// One block = one 512-key tile of one unit (batch, KV head), for all G query
// heads of that KV head.  Blocks are small and many so that the hardware
// keeps several per compute unit and balances them dynamically.  With SP > 1
// a block takes up to SP consecutive tiles whose sampled keys come from the
// bucket lookup's bitmaps (their lists concatenated, one set of attention
// rounds, one record).
//
// Scan: lane l of wave w reads 16 bytes (8 keys) of the codes of tables w,
// w+4, w+8, ... (non-temporal loads, eight rows in flight) and counts, for
// every head, the tables whose code differs from the query's (xor, packed
// min with 1, add: two keys per 32-bit word, two tables per add).  Each wave
// turns its counts into "at least one" / "at least two of my tables
// matched" flags; combined through LDS, key i is sampled for head h when some
// wave has two matches or two waves have one (at least two of L tables).
// Forced keys (the static head/tail ranges) are sampled for every head with
// P = 1.
//
// Tiles covered by the bit-plane index (threshold 2) are scanned there
// instead: lane j of each 16-lane group holds word j (32 keys) of one table
// stream's planes, a table's mismatch word per head is the OR over its K
// planes of the plane XOR the query's bit, and "at least one / two matching
// tables" are bit masks, folded over the 16 streams through LDS.
//
// Compaction: wave ballots + popcounts rank the keys, giving the tile's
// union list (key, head mask) in LDS in ascending key order.
//
// Attention (Equations 9-11), in rounds of up to ATT_E list entries:
//  (a) each 16-lane group gathers two entries' key and value rows (8
//      elements per lane, all four loads in flight), stages the value rows in
//      LDS, reduces q_h.k and |k - mu|^2, and its lanes form the log-weights
//      s - ln P per (entry, head), or -inf where the head did not sample the
//      key;
//  (b) after one barrier, one thread per (head, dims) folds the round into
//      its running maximum m, normaliser l and unnormalised output o (online
//      softmax).
// The query codes, queries and key mean are fetched while the first batch
// of codes is in flight.  One partial record (m, l, count, o) per head.
template <typename T, int GM, int SP>
__global__ __launch_bounds__(256, (GM <= 4 ? (sizeof(T) == 2 ? MP_OCC : MP_OCC_F32) : MP_OCC8)) void sample_kernel(
    const T *__restrict__ q, const T *__restrict__ Kc, const T *__restrict__ Vc, const uint16_t *__restrict__ codes,
    const float *__restrict__ kmean, const uint16_t *__restrict__ qcodes, int Hq, int Hkv, int G, int64_t n,
    int64_t cap, int K, int L, int64_t nsh, int64_t nst, int64_t nchunks, float scale, uint32_t one2, LnPCoef cf,
    float *__restrict__ part, uint32_t *__restrict__ ent, int32_t *__restrict__ ent_cnt,
    const uint32_t *__restrict__ planes, int64_t npt, int64_t ptiles, const uint32_t *__restrict__ sbits,
    int64_t bwords, int64_t nlt, const float *__restrict__ rlift, int nunits) {
  // Per-wave match flags of the lane's 8 keys for every head: bit h*8+k of
  // words [0, FW) says "at least one of this wave's tables matched", of
  // words [FW, 2FW) "at least two".
  constexpr int FW = (GM * 8 + 31) / 32;
  struct ScanLds {
    uint32_t flg[4][64][2 * FW];
  };
  struct CntLds {  // thresholds other than 2: per-wave match counts [wave][lane][key][head]
    uint8_t c[4][64][8][GM];
  };
  struct AttnLds {
    T v[ATT_E][D];                         // staged value rows of this round's entries
    alignas(16) float lw[GM][ATT_E];       // log-weights s - ln P (or -inf), head-major
  };
  struct PlaneLds {  // per table stream: "at least one" / "at least two" words [stream][head][word]
    uint32_t c1[16][GM][16];
    uint32_t c2[16][GM][16];
  };
  struct MfmaLds {  // matrix-core rounds (bf16 caches)
    alignas(16) __bf16 vT[D][VT_STRIDE];  // value rows transposed: [dim][entry]
    // exp(w - m) per head and entry as two bf16 parts (hi + lo: 16
    // significant bits); row GM zero (the padding heads' row)
    alignas(16) __bf16 ph[GM + 1][ATT_E];
    alignas(16) __bf16 pl[GM + 1][ATT_E];
    float sdot[2][GM][ATT_E];             // q_h . k per head and entry: dims 0-63, 64-127
    float nrm[2][ATT_E];                  // |k - mu|^2 per entry: dims 0-63, 64-127
  };
  __shared__ union {
    ScanLds s;
    CntLds c;
    AttnLds a;
    PlaneLds p;
    MfmaLds m;
  } sm;  // scan and attention phases never overlap in time
  // per head, a tile's sampled-key words: the bucket lookup's bitmaps of the
  // block's tiles, or the plane scan's result
  __shared__ uint32_t pw2[SP][GM][16];
  extern __shared__ u32x4 qpk4[];  // [L][GM] query codes, each twice per word (16-byte aligned)
  uint32_t *qpk = (uint32_t *)qpk4;
  // the queries in the caches' type; with bf16 caches they are the
  // matrix-core rounds' B operands as they stand, row GM (and the rows of
  // heads past G) zero: the padding columns
  __shared__ alignas(16) T qsh[std::is_same<T, __bf16>::value ? GM + 1 : GM][D];
  __shared__ float msh[D];
  // per head: |q_h|, q_h . mu, running maximum m, running normaliser l (one
  // 16-byte LDS word, so that the weight phase reads all four at once)
  __shared__ f32x4 hst[GM];
  // union list, read through lslot: key offset from the block's first key,
  // and head bits | FORCED.  One tile: a segment of up to 128 entries per wave
  // (the wave's 128 keys); several tiles: contiguous, tile after tile
  __shared__ uint16_t lkey[SP * SCAN_TILE];
  __shared__ uint16_t lmask[SP * SCAN_TILE];
  __shared__ int wtot[2][4];  // per wave: a tile's list entries (two buffers, alternating over the tiles)
  __shared__ int hcw[4][GM];  // per wave and head: sampled keys
  __shared__ float alpha_sh[GM];  // per head: this round's rescale factor

  touch_kernargs<5>();  // 292 bytes of arguments
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: table bases stay scalar
  const int j16 = lane & 15, grp = tid >> 4;
  // Blocks run tile-major: consecutive blocks take the same tile of
  // consecutive units, so the units' short last tiles are dispatched last and
  // are what a grid slightly larger than one round of blocks leaves over.
  // With bitmaps for the tiles below nlt, the tiles that still scan (the
  // appended keys past the bucketed tables: a few per unit, each a chain of
  // dependent load batches) are dispatched first, so their scans overlap the
  // other tiles' attention instead of trailing it.
  // A tile with bitmaps may share its block with the next ones: SP of them
  // per block (one prologue and fuller attention rounds, for grids many
  // times what the chip holds at once), the block's record in its first
  // tile's slot and empty records in the others.
  // (32-bit index arithmetic: a 64-bit division is a long instruction chain)
  const uint32_t bx = blockIdx.x, U32 = (uint32_t)nunits;
  const int64_t u = (int64_t)(bx % U32);
  const int64_t cr = (int64_t)(bx / U32), nscan = nchunks - nlt;
  const int64_t c = cr < nscan ? nlt + cr : (cr - nscan) * SP;  // the block's (first) tile
  const int nsub = (SP == 1 || c >= nlt) ? 1 : (int)min((int64_t)SP, nlt - c);  // its tiles
  const int b = (int)u / Hkv, kvh = (int)u % Hkv;
  const int64_t qrow0 = (int64_t)b * Hq + (int64_t)kvh * G;  // first query head of this unit
  // keys hashed lifted (Equation 8): the sampling angle is taken against the
  // lifted key, whose norm is the unit's radius (0: not lifted)
  const float rl = rlift ? rlift[u] : 0.0f;
  const int64_t tbase = c * SCAN_TILE;
  const int64_t tend = min(n, tbase + SCAN_TILE);
  const uint16_t headbits = (uint16_t)((1u << G) - 1u);
  const u16x2 one = __builtin_bit_cast(u16x2, one2);

  // This wave's tables are wave, wave+4, ...  A lane reads 16 bytes (8 keys)
  // per table row: a batch of MP_SB rows is read through a buffer resource
  // based at the batch's first row, with the row's offset in a scalar and the
  // lane's in a vector register (no per-row address arithmetic).  Loads are
  // unconditional: lanes past the last key re-read the tile's first 8 keys
  // and tables past the wave's last re-read its last table (all inside the
  // code store; their counts are discarded).  The code store is streamed
  // once: non-temporal loads keep it from evicting the caches' reused lines
  // (query codes, keys and values of the list).
  const int ntw = (L - wave + 3) / 4;
  const int jlast = ntw - 1;
  const int64_t rstride = 8 * cap;  // bytes between this wave's consecutive tables
  const uint32_t rstride32 = (uint32_t)rstride;  // MP_SB rows span < 2^32 bytes (cap < 2^26)
  const char *rows0 = (const char *)(codes + u * (int64_t)L * cap + (int64_t)wave * cap + tbase);
  const uint32_t lo = (tbase + 8 * lane < tend) ? 16u * (uint32_t)lane : 0u;
  uint4 cw[MP_SB];
  // rows j0 + hf*MP_SB/2 .. + MP_SB/2 - 1 (clamped to the last) into cw's half hf
  auto load_half = [&](int j0, int hf) {
    const int jb = min(j0 + hf * (MP_SB / 2), jlast);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(rows0 + (int64_t)jb * rstride), 0, -1, 0x00020000);
#pragma unroll
    for (int r = 0; r < MP_SB / 2; ++r)
      cw[hf * (MP_SB / 2) + r] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     rs, lo, (uint32_t)(min(j0 + hf * (MP_SB / 2) + r, jlast) - jb) * rstride32, 2));
  };
  // Tiles below nlt take their sampled keys from the bucket lookup's bitmaps;
  // tiles the bit-plane index covers are scanned there (threshold 2 only).
  const bool use_bits = c < nlt;
  const bool use_pl = !use_bits && planes != nullptr && K > 0 && cf.T == 2 && c < npt;
  // A narrow tile (at most 256 keys: the appended keys past an index, a
  // short last tile) needs fewer than 64 lanes per table row: P = 2^lgp lanes
  // (one per group of 8 keys) read a row, so a wave reads S = 64 / P of its
  // rows per load -- rows j0 + slot + S r -- and its chain of dependent load
  // batches shrinks S-fold.  The lanes of one key group add their mismatch
  // counts at the end.
  const int nkg = (int)((tend - tbase + 7) >> 3);
  const bool narrow = nkg <= 32;
  const int lgp = !narrow ? 6 : nkg <= 1 ? 0 : 32 - __builtin_clz((unsigned)(nkg - 1));
  const int nslot = 64 >> lgp, slot = lane >> lgp, kgrp = lane & ((1 << lgp) - 1);
  const int64_t nlo = (tbase + 8 * kgrp < tend) ? 16 * kgrp : 0;
  auto load_narrow = [&](int j0) {
#pragma unroll
    for (int r = 0; r < MP_SB; ++r)
      if (j0 + nslot * r < ntw)  // uniform: some lane of the wave still has a row here
        cw[r] = *(const uint4 *)(rows0 + (int64_t)min(j0 + slot + nslot * r, jlast) * rstride + nlo);
  };
  if (!use_bits && !use_pl && ntw > 0) {
    if (narrow) {
      load_narrow(0);
    } else {
      load_half(0, 0);
      load_half(0, 1);
    }
  }
  // tiles with bitmaps: their words of every head, loaded with the prologue's loads
  uint32_t bword[SP];
#pragma unroll
  for (int t = 0; t < SP; ++t) {
    bword[t] = 0u;
    if (use_bits && t < nsub && tid < GM * 16 && (tid >> 4) < G)
      bword[t] = sbits[(u * G + (tid >> 4)) * bwords + (c + t) * 16 + (tid & 15)];
  }

  // ---- prologue: query codes (packed twice per word), queries, key mean.
  // Every load of a pass is issued before any is used (one memory round trip
  // instead of one per element); indices past the end re-read a valid
  // element and are not stored.
  constexpr int QPASS = 4;                     // query-code loads per thread and pass
  constexpr int QV = (GM * D + 255) / 256;     // query elements per thread
  {
    const int nq = use_bits ? 0 : L * GM;  // a tile with bitmaps needs no query codes
    int i0 = tid;
    do {
      uint16_t cq[QPASS];
      T qv[QV];
      float mv = 0.0f;
      if (nq > 0) {
#pragma unroll
        for (int k = 0; k < QPASS; ++k) {
          const int i = min(i0 + 256 * k, nq - 1), l = i / GM, h = min(i % GM, G - 1);
          cq[k] = qcodes[(qrow0 + h) * L + l];
        }
      }
      const bool first = i0 == tid;
      if (first) {
#pragma unroll
        for (int k = 0; k < QV; ++k) {
          const int i = min(tid + 256 * k, GM * D - 1), h = min(i / D, G - 1);
          qv[k] = q[(qrow0 + h) * D + i % D];
        }
        mv = kmean[u * D + (tid & (D - 1))];
      }
      __builtin_amdgcn_sched_barrier(0);  // keeps the loads ahead of every use
#pragma unroll
      for (int k = 0; k < QPASS; ++k) {
        const int i = i0 + 256 * k;
        if (i < nq) {
          const uint32_t code = i % GM < G ? (uint32_t)cq[k] : 0u;
          qpk[i] = code | (code << 16);
        }
      }
      if (first) {
#pragma unroll
        for (int k = 0; k < QV; ++k) {
          const int i = tid + 256 * k;
          if (i < GM * D) qsh[i / D][i % D] = i / D < G ? qv[k] : (T)0.0f;
        }
        if (tid < D) msh[tid] = mv;
        if constexpr (std::is_same<T, __bf16>::value) {
          if (tid < D) qsh[GM][tid] = (T)0.0f;
        }
      }
      i0 += 256 * QPASS;
    } while (i0 < nq);
  }
  if (tid < GM) {
    hst[tid][2] = -INFINITY;
    hst[tid][3] = 0.0f;
  }
  if (tid < GM * 16) {
#pragma unroll
    for (int t = 0; t < SP; ++t) pw2[t][tid >> 4][tid & 15] = bword[t];
  }
  __syncthreads();

  if (tid < 16 * GM) {  // |q_h| and q_h . mu: a DPP row (16 lanes, 8 dims each) per head
    const int h = tid >> 4;
    float qv[8], mv[8];
    ld8<T>(&qsh[h][8 * j16], qv);
    ld8<float>(msh + 8 * j16, mv);
    float a = 0.0f, bq = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a = fmaf(qv[e], qv[e], a);
      bq = fmaf(qv[e], mv[e], bq);
    }
    a = row16_sum(a);
    bq = row16_sum(bq);
    if (j16 == 0) {
      hst[h][0] = sqrtf(a);
      hst[h][1] = bq;
    }
  }

  int nu = 0;  // entries in the union list
  int lp1 = 0, lp2 = 0, lp3 = 0;  // one tile per block: list entries before waves 1, 2, 3's segments
  // LDS slot of list entry e.  One tile per block: the list is the waves'
  // segments in wave order (ascending keys); branch-free, each segment
  // boundary passed adds the gap to the next segment's start.  Several
  // tiles: the list is contiguous.
  auto lslot = [&](int e) {
    if constexpr (SP > 1) {
      return e;
    } else {
      return e + (e >= lp1 ? 128 - lp1 : 0) + (e >= lp2 ? 128 + lp1 - lp2 : 0) + (e >= lp3 ? 128 + lp2 - lp3 : 0);
    }
  };
  uint32_t *uent = ent ? ent + (u * nchunks + c) * (2 * SCAN_TILE) : nullptr;
  {
    // query codes of table l for every head (GM >= 4: 16-byte LDS reads)
    auto qcodes_of = [&](int l, uint32_t (&Q)[GM]) {
      if constexpr (GM >= 4) {
#pragma unroll
        for (int k = 0; k < GM / 4; ++k) {
          const u32x4 v = qpk4[l * (GM / 4) + k];
          Q[4 * k] = v[0];
          Q[4 * k + 1] = v[1];
          Q[4 * k + 2] = v[2];
          Q[4 * k + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int h = 0; h < GM; ++h) Q[h] = qpk[l * GM + h];
      }
    };
    uint32_t mlo = 0, mhi = 0;  // keys 2*tid, 2*tid+1 of the tile: heads that sampled them
    if (use_bits) {
      // decoded per tile below
    } else if (use_pl) {
      // Bit-plane scan: the tile's planes are one contiguous region, row
      // (b, l) = bit b of table l's codes for the tile's 512 keys (16 words).
      // Lane j of a 16-lane group holds word j (32 keys); the wave's four
      // groups take four consecutive tables (one contiguous 256-byte read per
      // plane).  Per head, the 32 keys' mismatch word of a table is the OR over
      // b of the plane XOR the query's bit b (sign-extended); "at least one" /
      // "at least two" matching tables are kept as bit masks.
      const int pj = lane & 15, sg = (wave << 2) | (lane >> 4);  // word, table stream
      const uint32_t *pt = planes + (u * ptiles + c) * (int64_t)K * L * 16 + pj;
      uint32_t c1[GM], c2[GM];
#pragma unroll
      for (int h = 0; h < GM; ++h) c1[h] = c2[h] = 0u;
      // KB >= K planes per table; planes past K repeat plane K-1 (same word,
      // same query bit), which leaves the OR unchanged
      auto pscan = [&](auto kbc) {
        constexpr int KB = decltype(kbc)::value;
        for (int l = sg; l < L; l += 16) {
          uint32_t pw[KB];
#pragma unroll
          for (int b = 0; b < KB; ++b) pw[b] = __builtin_nontemporal_load(pt + ((int64_t)min(b, K - 1) * L + l) * 16);
          uint32_t Q[GM];
          qcodes_of(l, Q);
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            uint32_t m = 0u;
#pragma unroll
            for (int b = 0; b < KB; ++b) m |= pw[b] ^ (uint32_t)__builtin_amdgcn_sbfe((int)Q[h], min(b, K - 1), 1);
            c2[h] |= c1[h] & ~m;
            c1[h] |= ~m;
          }
        }
      };
      if (K <= 8)
        pscan(std::integral_constant<int, 8>{});
      else if (K <= 10)
        pscan(std::integral_constant<int, 10>{});
      else if (K <= 12)
        pscan(std::integral_constant<int, 12>{});
      else
        pscan(std::integral_constant<int, 16>{});
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        sm.p.c1[sg][h][pj] = c1[h];
        sm.p.c2[sg][h][pj] = c2[h];
      }
      __syncthreads();
      if (tid < GM * 16) {  // fold the 16 streams: at least two overall
        const int h = tid >> 4, jj = tid & 15;
        uint32_t a1 = 0u, a2 = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t b1 = sm.p.c1[v][h][jj], b2 = sm.p.c2[v][h][jj];
          a2 |= b2 | (a1 & b1);
          a1 |= b1;
        }
        pw2[0][h][jj] = h < G ? a2 : 0u;
      }
      __syncthreads();
      const int wj = tid >> 4, k0 = (2 * tid) & 31;  // keys 2*tid, 2*tid+1: word wj, bits k0, k0+1
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        const uint32_t wv = pw2[0][h][wj];
        mlo |= ((wv >> k0) & 1u) << h;
        mhi |= ((wv >> (k0 + 1)) & 1u) << h;
      }
    } else {
    // ---- scan
    uint32_t acc[GM][4];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[h][w] = 0;
#define MP_MIS(word, Q) \
  __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, (word) ^ (Q)), one))
    // two tables (rows ra, rb: tables l and l + 4) into the mismatch counts
    auto scan_pair = [&](const uint4 &ra, const uint4 &rb, int l) {
      const uint32_t a4[4] = {ra.x, ra.y, ra.z, ra.w};
      const uint32_t b4[4] = {rb.x, rb.y, rb.z, rb.w};
      if constexpr (GM == 8) {  // eight heads: one head's two codes live at a time (register budget)
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const uint32_t Qa = qpk[l * GM + h], Qb = qpk[(l + 4) * GM + h];
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] = acc[h][w] + MP_MIS(a4[w], Qa) + MP_MIS(b4[w], Qb);
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
        uint32_t Qa[GM], Qb[GM];
        qcodes_of(l, Qa);
        qcodes_of(l + 4, Qb);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] = acc[h][w] + MP_MIS(a4[w], Qa[h]) + MP_MIS(b4[w], Qb[h]);
          __builtin_amdgcn_sched_barrier(0);  // few temporaries live at once
        }
      }
    };
    if (narrow) {  // rows j0 + slot + S r of a batch; rows past the wave's last add no mismatch
      for (int j0 = 0; j0 < ntw; j0 += nslot * MP_SB) {
        if (j0 > 0) load_narrow(j0);
#pragma unroll
        for (int r = 0; r < MP_SB; ++r) {
          if (j0 + nslot * r >= ntw) break;  // uniform
          const int j = j0 + slot + nslot * r;
          const bool live = j < ntw;
          const int l = wave + 4 * min(j, jlast);
          uint32_t Qa[GM];
          if constexpr (GM != 8) qcodes_of(l, Qa);
          const uint32_t a4[4] = {cw[r].x, cw[r].y, cw[r].z, cw[r].w};
#pragma unroll
          for (int h = 0; h < GM; ++h) {
            const uint32_t Q = GM == 8 ? qpk[l * GM + h] : Qa[h];
#pragma unroll
            for (int w = 0; w < 4; ++w)
              acc[h][w] += live ? __builtin_bit_cast(uint32_t, __builtin_elementwise_min(
                                                                   __builtin_bit_cast(u16x2, a4[w] ^ Q), one))
                                : 0u;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // the slots of a key group hold disjoint tables: add their counts (two
      // 16-bit counts per word, each at most the wave's table count)
      for (int sh = 1 << lgp; sh < 64; sh <<= 1)
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] += (uint32_t)__shfl_xor((int)acc[h][w], sh);
    }
    // whole batches (branch-free pairs), then the wave's last, partial batch
    // outside the loop (one code path per loop body keeps the counts in one
    // set of registers)
    // Two halves per batch: the next batch's half is issued as soon as this
    // half's rows have been counted, so a wave keeps loads in flight while
    // it computes.
    int j0 = narrow ? ntw : 0;
    for (; j0 + MP_SB <= ntw; j0 += MP_SB) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int jj = hf * (MP_SB / 2); jj < (hf + 1) * (MP_SB / 2); jj += 2) {
          scan_pair(cw[jj], cw[jj + 1], wave + 4 * (j0 + jj));
          // one pair's query codes live at a time
          __builtin_amdgcn_sched_barrier(0);
        }
        load_half(j0 + MP_SB, hf);
      }
    }
    if (j0 < ntw) {  // rows already loaded; tables past the wave's last add no mismatch (selects)
#pragma unroll
      for (int jj = 0; jj < MP_SB; ++jj) {
        const bool live = j0 + jj < ntw;
        const int l = min(wave + 4 * (j0 + jj), L - 1);
        uint32_t Qa[GM];
        if constexpr (GM != 8) qcodes_of(l, Qa);
        const uint32_t a4[4] = {cw[jj].x, cw[jj].y, cw[jj].z, cw[jj].w};
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const uint32_t Q = GM == 8 ? qpk[l * GM + h] : Qa[h];
#pragma unroll
          for (int w = 0; w < 4; ++w) acc[h][w] += live ? MP_MIS(a4[w], Q) : 0u;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
#undef MP_MIS
    {  // this wave's matches per (key, head) -> "at least one" / "at least two" flags
      uint32_t g1[FW], g2[FW];
#pragma unroll
      for (int f = 0; f < FW; ++f) g1[f] = g2[f] = 0;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int mlo = ntw - (int)(acc[h][w] & 0xffffu), mhi = ntw - (int)(acc[h][w] >> 16);
          const int bit = h * 8 + 2 * w;  // keys 2w (low half) and 2w+1 (high half)
          g1[bit >> 5] |= ((uint32_t)(mlo >= 1) | ((uint32_t)(mhi >= 1) << 1)) << (bit & 31);
          g2[bit >> 5] |= ((uint32_t)(mlo >= 2) | ((uint32_t)(mhi >= 2) << 1)) << (bit & 31);
        }
      }
      if (cf.T == 2) {
#pragma unroll
        for (int f = 0; f < FW; ++f) {
          sm.s.flg[wave][lane][f] = g1[f];
          sm.s.flg[wave][lane][FW + f] = g2[f];
        }
      } else {  // other thresholds: this wave's match counts (<= 128 tables per wave)
#pragma unroll
        for (int h = 0; h < GM; ++h)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            sm.c.c[wave][lane][2 * w][h] = (uint8_t)(ntw - (int)(acc[h][w] & 0xffffu));
            sm.c.c[wave][lane][2 * w + 1][h] = (uint8_t)(ntw - (int)(acc[h][w] >> 16));
          }
      }
    }
    __syncthreads();

    // ---- threshold + compaction: thread tid owns sub-tile keys 2*tid, 2*tid+1
    // (scan lane tid/4, key slots k0 = 2*(tid%4) and k0+1).  At least two
    // matching tables overall <=> some wave has two, or two waves have one;
    // any other threshold adds the four waves' counts.
    if (cf.T != 2) {
      const int sl = tid >> 2, k0 = 2 * (tid & 3);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const int s0 = sm.c.c[0][sl][k0][h] + sm.c.c[1][sl][k0][h] + sm.c.c[2][sl][k0][h] + sm.c.c[3][sl][k0][h];
          const int s1 = sm.c.c[0][sl][k0 + 1][h] + sm.c.c[1][sl][k0 + 1][h] + sm.c.c[2][sl][k0 + 1][h] +
                         sm.c.c[3][sl][k0 + 1][h];
          mlo |= (uint32_t)(s0 >= cf.T) << h;
          mhi |= (uint32_t)(s1 >= cf.T) << h;
        }
      }
    } else {
      const int sl = tid >> 2, k0 = 2 * (tid & 3);
#pragma unroll
      for (int f = 0; f < FW; ++f) {
        const uint32_t a1 = sm.s.flg[0][sl][f], b1 = sm.s.flg[1][sl][f], c1 = sm.s.flg[2][sl][f],
                       d1 = sm.s.flg[3][sl][f];
        const uint32_t two = sm.s.flg[0][sl][FW + f] | sm.s.flg[1][sl][FW + f] | sm.s.flg[2][sl][FW + f] |
                             sm.s.flg[3][sl][FW + f] | (a1 & (b1 | c1 | d1)) | (b1 & (c1 | d1)) | (c1 & d1);
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          if ((h * 8) >> 5 == f && h < G) {
            mlo |= ((two >> ((h * 8 + k0) & 31)) & 1u) << h;
            mhi |= ((two >> ((h * 8 + k0 + 1) & 31)) & 1u) << h;
          }
        }
      }
    }
    }
    for (int t = 0; t < nsub; ++t) {
      const int64_t tb = tbase + t * SCAN_TILE, te = min(n, tb + SCAN_TILE);
      const int64_t klo = tb + 2 * tid;
      if (use_bits) {
        // the tile's sampled-key words of every head, as the bucket lookup
        // wrote them (staged with the prologue)
        const int wj = tid >> 4, k0 = (2 * tid) & 31;  // keys 2*tid, 2*tid+1: word wj, bits k0, k0+1
        mlo = mhi = 0u;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
          const uint32_t wv = pw2[t][h][wj];
          mlo |= ((wv >> k0) & 1u) << h;
          mhi |= ((wv >> (k0 + 1)) & 1u) << h;
        }
      }
      if (klo < nsh || klo >= n - nst) mlo = headbits | FORCED;
      if (klo + 1 < nsh || klo + 1 >= n - nst) mhi = headbits | FORCED;
      if (klo >= te) mlo = 0;
      if (klo + 1 >= te) mhi = 0;
      const bool flo = (mlo & headbits) != 0, fhi = (mhi & headbits) != 0;
      const uint64_t blo = __ballot(flo), bhi = __ballot(fhi);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int pre = __popcll(blo & lt) + __popcll(bhi & lt);
      if (lane == 0) wtot[t & 1][wave] = __popcll(blo) + __popcll(bhi);
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          const int ch = __popcll(__ballot((mlo >> h) & 1)) + __popcll(__ballot((mhi >> h) & 1));
          if (lane == 0) hcw[wave][h] = (t > 0 ? hcw[wave][h] : 0) + ch;
        }
      }
      const int kloc = (int)(klo - tbase);  // offset from the block's first key
      if constexpr (SP == 1) {
        // each wave writes its own segment (no offsets across waves needed yet)
        const int sb = 128 * wave + pre;
        if (flo) {
          lkey[sb] = (uint16_t)kloc;
          lmask[sb] = (uint16_t)mlo;
        }
        if (fhi) {
          lkey[sb + (flo ? 1 : 0)] = (uint16_t)(kloc + 1);
          lmask[sb + (flo ? 1 : 0)] = (uint16_t)mhi;
        }
        __syncthreads();  // list complete
        lp1 = wtot[0][0];
        lp2 = lp1 + wtot[0][1];
        lp3 = lp2 + wtot[0][2];
        nu = lp3 + wtot[0][3];
        if (uent) {  // the index list in key order
          const int off = (wave == 0 ? 0 : wave == 1 ? lp1 : wave == 2 ? lp2 : lp3) + pre;
          if (flo) uent[off] = (uint32_t)kloc | ((mlo & headbits) << 16);
          if (fhi) uent[off + (flo ? 1 : 0)] = (uint32_t)(kloc + 1) | ((mhi & headbits) << 16);
        }
      } else {
        // the tile's entries follow the earlier tiles' (the wave counts go
        // through LDS, in two buffers that alternate over the tiles)
        __syncthreads();
        const int w0 = wtot[t & 1][0], w1 = wtot[t & 1][1], w2 = wtot[t & 1][2], w3 = wtot[t & 1][3];
        const int off = nu + (wave > 0 ? w0 : 0) + (wave > 1 ? w1 : 0) + (wave > 2 ? w2 : 0) + pre;
        if (flo) {
          lkey[off] = (uint16_t)kloc;
          lmask[off] = (uint16_t)mlo;
          if (uent) uent[off] = (uint32_t)kloc | ((mlo & headbits) << 16);
        }
        if (fhi) {
          const int o2 = off + (flo ? 1 : 0);
          lkey[o2] = (uint16_t)(kloc + 1);
          lmask[o2] = (uint16_t)mhi;
          if (uent) uent[o2] = (uint32_t)(kloc + 1) | ((mhi & headbits) << 16);
        }
        nu += w0 + w1 + w2 + w3;
      }
    }
    if constexpr (SP > 1) __syncthreads();  // list complete
  }
  if (ent_cnt && tid < nsub) ent_cnt[u * nchunks + c + tid] = tid == 0 ? nu : 0;

  // ---- attention over the union list
  if constexpr (std::is_same<T, __bf16>::value) {
    // Matrix-core rounds of ATT_E entries (16x16x32 bf16 operations, fp32
    // accumulation; heads padded to 16 columns):
    //  (a) wave w gathers half of the rows of 16 entries: entries
    //      16 (w & 1) + li, dims 64 (w >> 1) .. + 63, lane (qd, li) holding dims
    //      32 s + 8 qd .. + 7 of its two 32-dim steps s -- the A-operand
    //      layout -- so its half of S = K Q^T takes two operations; lanes also
    //      sum |k - mu|^2 over their 16 dims (fp32) and stage the value rows
    //      transposed ([dim][entry]) in LDS; the two halves meet in (b);
    //  (b) one thread per (head, entry) forms the log-weight
    //      s = q.k / sqrt(d) - ln P (or -inf where the head did not sample the
    //      key), the head's new running maximum m (a 32-lane max), exp(s - m)
    //      -- stored as two bf16 parts (hi + lo, 16 significant bits) so the
    //      weights keep fp32-like precision -- and the round's sum, and
    //      records m, the rescale factor and the running normaliser;
    //  (c) wave w accumulates the output dims 32 w .. 32 w + 31 of every head
    //      as O = O * alpha + P V (P's two parts, two operations each).
    const int qd = lane >> 4, li = lane & 15;
    f32x4 oacc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};  // heads 4 qd + j, dim 16 (2 wave + b) + li
    // the block's rows (scalar bases) and a lane's 32-bit byte offsets from
    // them (the rows of up to SP tiles: below 2^20 bytes), so no lane holds a
    // 64-bit pointer
    const char *Kb = (const char *)((const __bf16 *)Kc + (u * cap + tbase) * D);
    const char *Vb = (const char *)((const __bf16 *)Vc + (u * cap + tbase) * D);
    // this lane's key and value pieces of the round starting at entry r0
    // (r0 < nu).  Slots past the list read the list's last key again: a
    // sampled key's rows, whose dot products are dropped and whose value rows
    // meet weight 0 (finite, so the products are exact zeros)
    uint4 kr[2], vr[2];
    auto load_round = [&](int r0) {
      const int e = 16 * (wave & 1) + li, kh = wave >> 1;
      const uint32_t key = lkey[lslot(r0 + min(e, nu - r0 - 1))];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const uint32_t bo = 2u * (key * D + 8u * qd + 64u * kh + 32u * st);
        kr[st] = *(const uint4 *)(Kb + bo);
        vr[st] = *(const uint4 *)(Vb + bo);
      }
    };
    // With four or more heads per block, or several tiles (several rounds),
    // the next round's rows are requested as soon as this round's are
    // consumed (end of (a)), so they arrive while (b) and (c) run (the
    // barriers wait for LDS operations only); with one tile of fewer heads
    // (short (b) and (c), many blocks) at the start of the round.
    constexpr bool early = GM >= 4 || SP > 1;
    if (tid < ATT_E) {  // the padding heads' weights (no phase writes this row)
      sm.m.ph[GM][tid] = (__bf16)0.0f;
      sm.m.pl[GM][tid] = (__bf16)0.0f;
    }
    if (nu > 0) load_round(0);
    for (int e0 = 0; e0 < nu; e0 += ATT_E) {
      const int ne = min(ATT_E, nu - e0);
      if (!early && e0 > 0) load_round(e0);
      {  // (a)
        const int e = 16 * (wave & 1) + li, kh = wave >> 1;

        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
        float n2 = 0.0f;
        const int hq = li < G ? li : GM;  // row GM: zeros
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const int d0 = 64 * kh + 32 * st + 8 * qd;
          const bf16x8 kb = __builtin_bit_cast(bf16x8, kr[st]);
          float mv[8];
          ld8<float>(msh + d0, mv);
          const bf16x8 qb = *(const bf16x8 *)&qsh[hq][d0];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float cj = (float)kb[j] - mv[j];
            n2 += cj * cj;
          }
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, sacc, 0, 0, 0);
        }
        n2 += swz_xor<16>(n2);
        n2 += __shfl_xor(n2, 32);
        if (li < GM) {
#pragma unroll
          for (int j = 0; j < 4; ++j) sm.m.sdot[kh][li][16 * (wave & 1) + 4 * qd + j] = sacc[j];
        }
        if (qd == 0) sm.m.nrm[kh][e] = n2;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 vb = __builtin_bit_cast(bf16x8, vr[st]);
#pragma unroll
          for (int j = 0; j < 8; ++j) sm.m.vT[64 * kh + 32 * st + 8 * qd + j][e] = vb[j];
        }
        if (early && e0 + ATT_E < nu) load_round(e0 + ATT_E);
      }
      __syncthreads();
      if (tid < GM * ATT_E) {  // (b)
        const int h = tid / ATT_E, e = tid % ATT_E;
        const f32x4 hs = hst[h];
        float w = -INFINITY;
        if (h < G && e < ne) {
          const uint32_t mk = lmask[lslot(e0 + e)];
          if ((mk >> h) & 1u) {
            const float dk = sm.m.sdot[0][h][e] + sm.m.sdot[1][h][e];
            float lnP = 0.0f;
            if (!(mk & FORCED)) {
              const float den = hs[0] * (rl > 0.0f ? rl : __builtin_amdgcn_sqrtf(sm.m.nrm[0][e] + sm.m.nrm[1][e]));
              const float cosv = den > 0.0f ? (dk - hs[1]) * __builtin_amdgcn_rcpf(den) : 0.0f;
              lnP = log_sampling_prob(cosv, K, L, cf);
            }
            w = dk * scale - lnP;
          }
        }
        const float mr = xor32_max(w);  // within the 32 lanes of h
        const float mo = hs[2];
        const float mn = fmaxf(mo, mr);
        const float pe = mn > -INFINITY ? hw_exp(w - mn) : 0.0f;  // 0 for -inf
        const float ps = xor32_sum(pe);
        const __bf16 phi = (__bf16)pe;  // 0 for the heads past G
        sm.m.ph[h][e] = phi;
        sm.m.pl[h][e] = (__bf16)(pe - (float)phi);
        if (e == 0) {
          const float alpha = mn > -INFINITY ? hw_exp(mo - mn) : 1.0f;  // 0 while mo = -inf
          alpha_sh[h] = alpha;
          hst[h][2] = mn;
          hst[h][3] = hs[3] * alpha + ps;
        }
      }
      __syncthreads();
      {  // (c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int h = 4 * qd + j;
          const float a = h < GM ? alpha_sh[h < GM ? h : 0] : 1.0f;
          oacc[0][j] *= a;
          oacc[1][j] *= a;
        }
        const int hr = li < GM ? li : GM;
        const bf16x8 ph = *(const bf16x8 *)&sm.m.ph[hr][8 * qd];
        const bf16x8 pl = *(const bf16x8 *)&sm.m.pl[hr][8 * qd];
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2) {
          const bf16x8 vb = *(const bf16x8 *)&sm.m.vT[16 * (2 * wave + b2) + li][8 * qd];
          oacc[b2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vb, oacc[b2], 0, 0, 0);
          oacc[b2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, oacc[b2], 0, 0, 0);
        }
      }
      if (e0 + ATT_E < nu) __syncthreads();  // the next round reuses the staging
    }
    float *rec0 = part + (u * nchunks + c) * G * PSTRIDE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int h = 4 * qd + j;
      if (h < G) {
        rec0[h * PSTRIDE + 4 + 16 * (2 * wave) + li] = oacc[0][j];
        rec0[h * PSTRIDE + 4 + 16 * (2 * wave + 1) + li] = oacc[1][j];
      }
    }
    if (tid < G) {
      float *rec = rec0 + tid * PSTRIDE;
      rec[0] = hst[tid][2];
      rec[1] = hst[tid][3];
      rec[2] = __builtin_bit_cast(float, hcw[0][tid] + hcw[1][tid] + hcw[2][tid] + hcw[3][tid]);
      rec[3] = 0.0f;
    }
    if constexpr (SP > 1) {  // the block's other tiles: empty records (m = -inf, l = 0, count 0)
      if (tid < G * (nsub - 1)) *(f32x4 *)(rec0 + (G + tid) * PSTRIDE) = f32x4{-INFINITY, 0.0f, 0.0f, 0.0f};
    }
    return;
  }
  constexpr int TPH = (256 / GM) < 128 ? (256 / GM) : 128;  // output threads per head
  constexpr int DPT = D / TPH;                              // dims per output thread
  const int oh = tid / TPH, od = (tid % TPH) * DPT;
  const bool othread = oh < G && tid < GM * TPH;
  float ol = 0.0f, oacc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) oacc[i] = 0.0f;
  const T *Ku = Kc + (u * cap + tbase) * D + 8 * j16;
  const T *Vu = Vc + (u * cap + tbase) * D + 8 * j16;
  for (int e0 = 0; e0 < nu; e0 += ATT_E) {
    const int ne = min(ATT_E, nu - e0);
    static_assert(ATT_E == 32, "two entries per 16-lane group");
    const int el0 = grp, el1 = grp + 16;
    if (el0 < ne) {  // (a) gather both entries, then dots and log-weights
      const bool ok1 = el1 < ne;
      Raw8<T> k0, v0, k1, v1;
      const int64_t key0 = lkey[lslot(e0 + el0)];
      k0.load(Ku + key0 * D);
      v0.load(Vu + key0 * D);
      uint32_t mk1 = 0;
      if (ok1) {
        const int64_t key1 = lkey[lslot(e0 + el1)];
        k1.load(Ku + key1 * D);
        v1.load(Vu + key1 * D);
        mk1 = lmask[lslot(e0 + el1)];
      } else {
        k1.zero();
        v1.zero();
      }
      entry_pair<T, GM>(k0, v0, k1, v1, ok1, el0, el1, lmask[lslot(e0 + el0)], mk1, j16, G, K, L, cf, scale, qsh, msh,
                        hst, sm.a.v, sm.a.lw, rl);
    }
    __syncthreads();
    // (b) one thread per (head, entry) turns the log-weights into
    // exp(w - m) against the head's new running maximum m (a 32-lane max),
    // in place, and one per head records m and the rescale factor of the
    // head's earlier rounds
    if (tid < GM * ATT_E) {
      const int h = tid / ATT_E, e = tid % ATT_E;
      const float x = (h < G && e < ne) ? sm.a.lw[h][e] : -INFINITY;
      float mr = x;
#pragma unroll
      for (int sh = ATT_E / 2; sh > 0; sh >>= 1) mr = fmaxf(mr, __shfl_xor(mr, sh));  // within the 32 lanes of h
      const float mo = hst[h][2];
      const float mn = fmaxf(mo, mr);
      if (h < G && e < ne) sm.a.lw[h][e] = mn > -INFINITY ? hw_exp(x - mn) : 0.0f;  // 0 for -inf
      if (e == 0) {
        alpha_sh[h] = mn > -INFINITY ? hw_exp(mo - mn) : 1.0f;  // 0 while mo = -inf
        hst[h][2] = mn;
      }
    }
    __syncthreads();
    // (c) each output thread folds the round into its head's normaliser l and
    // output slice o
    if (othread) {
      const float alpha = alpha_sh[oh];
      ol *= alpha;
#pragma unroll
      for (int i = 0; i < DPT; ++i) oacc[i] *= alpha;
      for (int el = 0; el < ne; el += 4) {
        const f32x4 p4 = *(const f32x4 *)&sm.a.lw[oh][el];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (el + k < ne) {
            const float pk = p4[k];
            ol += pk;
            float vv[DPT];
            ldv<T, DPT>(&sm.a.v[el + k][od], vv);
#pragma unroll
            for (int i = 0; i < DPT; ++i) oacc[i] += pk * vv[i];
          }
        }
      }
    }
    if (e0 + ATT_E < nu) __syncthreads();  // the next round reuses the staging
  }
  if (othread) {
    float *rec = part + ((u * nchunks + c) * G + oh) * PSTRIDE;
#pragma unroll
    for (int i = 0; i < DPT; ++i) rec[4 + od + i] = oacc[i];
    if (tid % TPH == 0) {
      rec[0] = hst[oh][2];
      rec[1] = ol;
      rec[2] = __builtin_bit_cast(float, hcw[0][oh] + hcw[1][oh] + hcw[2][oh] + hcw[3][oh]);
      rec[3] = 0.0f;
    }
  }
}

// --------------------------------------------------------------------------
// Bit-plane index of the code store (the same codes, K bits per key and table
// instead of 16): one block of 8 waves per (unit, tile, group of 8 tables),
// wave w taking table 8g + w.  Lane i holds the codes of keys 512 t + 64 c + i
// (c < 8, all eight loads in flight); the ballot of their bit b is bit b's
// plane for those 64 keys (two 32-key words), and lane b (b < K) of each lane
// half stores its half's word.
constexpr int PB_TABLES = 8;  // tables per plane-build block (one per wave)

__global__ __launch_bounds__(64 * PB_TABLES) void plane_build_kernel(const uint16_t *__restrict__ codes, int64_t cap,
                                                                     int K, int L, int64_t t0, int64_t nt,
                                                                     int64_t ptiles, uint32_t *__restrict__ planes) {
  const int ng = (L + PB_TABLES - 1) / PB_TABLES;
  const int64_t bid = blockIdx.x;
  const int g = (int)(bid % ng);
  const int64_t r = bid / ng;
  const int64_t t = t0 + r % nt, u = r / nt;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l = g * PB_TABLES + wave;
  if (l >= L) return;  // whole waves; the kernel has no barrier
  const uint16_t *src = codes + (u * L + l) * cap + t * SCAN_TILE + lane;
  uint32_t cd[SCAN_TILE / 64];
#pragma unroll
  for (int c = 0; c < SCAN_TILE / 64; ++c) cd[c] = src[64 * c];
  uint32_t *dst = planes + ((u * ptiles + t) * K * L + l) * 16 + (lane >> 5);
  const int bl = lane & 31;
#pragma unroll
  for (int c = 0; c < SCAN_TILE / 64; ++c) {
    uint32_t val = 0u;
    for (int b = 0; b < K; ++b) {
      const uint64_t bal = __ballot((cd[c] >> b) & 1u);
      if (bl == b) val = (uint32_t)(lane < 32 ? bal : bal >> 32);
    }
    if (bl < K) dst[(int64_t)bl * L * 16 + 2 * c] = val;
  }
}

hipError_t launch_plane_build(const uint16_t *codes, int64_t U, int64_t cap, int K, int L, int64_t t0, int64_t nt,
                              uint32_t *planes, hipStream_t s) {
  if (nt <= 0 || U <= 0) return hipSuccess;
  const int64_t ptiles = (cap + SCAN_TILE - 1) / SCAN_TILE;
  const int64_t nb = U * nt * ((L + PB_TABLES - 1) / PB_TABLES);
  plane_build_kernel<<<dim3((unsigned)nb), 64 * PB_TABLES, 0, s>>>(codes, cap, K, L, t0, nt, ptiles, planes);
  return hipGetLastError();
}

hipError_t launch_sample(int dtype, const void *q, const void *Kc, const void *Vc, const uint16_t *codes,
                         const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                         int K, int L, int Tthr, int64_t nsh, int64_t nst, const DecodeGeom &geo, const DecodeWs &ws,
                         bool want_idx, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop,
                         const uint32_t *planes, int64_t n_planes, int64_t n_lists, const float *rlift) {
  const int G = Hq / Hkv;
  const float scale = 1.0f / sqrtf((float)D);
  const uint32_t one2 = 0x00010001u;
  const LnPCoef cf = lnp_coef(K, L, Tthr);
  uint32_t *ent = want_idx ? ws.ent : nullptr;
  int32_t *ent_cnt = want_idx ? ws.ent_cnt : nullptr;
  const int64_t npt = planes ? n_planes / SCAN_TILE : 0;  // tiles the plane index covers
  const int64_t ptiles = (cap + SCAN_TILE - 1) / SCAN_TILE;
  const int64_t nlt = n_lists / SCAN_TILE;  // tiles whose sampled-key bitmaps the bucket lookup wrote
  // Bitmap tiles SPAN_TILES per block (bf16 caches, one or two query heads
  // per unit) when one tile per block would make a grid of at least
  // SPAN_MIN_BLOCKS blocks: four times what the chip keeps resident.
  const int span = sample_span(dtype, G, nlt, geo);
  const dim3 grid((unsigned)(geo.U * (geo.nchunks - nlt + (nlt + span - 1) / span)));
#define MP_SAMPLE(T, GMV, SPV)                                                                               \
  hipExtLaunchKernelGGL(sample_kernel<T, GMV, SPV>, grid, dim3(256), sizeof(uint32_t) * L * GMV, s, ev_start, ev_stop, 0, \
                        (const T *)q, (const T *)Kc, (const T *)Vc, codes, kmean, qcodes, Hq, Hkv, G, n, cap, K, L,  \
                        nsh, nst, geo.nchunks, scale, one2, cf, ws.part, ent, ent_cnt, planes, npt, ptiles, ws.bits, \
                        geo.nchunks_max * (SCAN_TILE / 32), nlt, rlift, (int)geo.U)
#define MP_SAMPLE_G(T)    \
  do {                    \
    if (G == 1)           \
      MP_SAMPLE(T, 1, 1); \
    else if (G == 2)      \
      MP_SAMPLE(T, 2, 1); \
    else if (G <= 4)      \
      MP_SAMPLE(T, 4, 1); \
    else                  \
      MP_SAMPLE(T, 8, 1); \
  } while (0)
  if (span > 1) {
    if (G == 1)
      MP_SAMPLE(__bf16, 1, SPAN_TILES);
    else
      MP_SAMPLE(__bf16, 2, SPAN_TILES);
  } else if (dtype == 0) {
    MP_SAMPLE_G(__bf16);
  } else {
    MP_SAMPLE_G(float);
  }
#undef MP_SAMPLE_G
#undef MP_SAMPLE
  return hipGetLastError();
}

}  // namespace mp
