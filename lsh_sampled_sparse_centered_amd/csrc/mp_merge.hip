// Log-sum-exp merge of the per-chunk partial results of the sampled decode
// attention (MagicPIG, arXiv 2410.16179v2, Section 4.4 "On-device cache":
// split attention whose splits are merged through their log-sum-exp).
#include <math.h>

#include "mp_internal.h"

namespace mp {

// --------------------------------------------------------------------------
// Log-sum-exp merge of the per-chunk partials of one query head (the
// recursive-attention merge of Section 4.4): with M = max_c m_c,
//   l = sum_c l_c e^{m_c - M},  out = sum_c o_c e^{m_c - M} / l,
//   lse = M + ln l.
// One block of 1024 threads per head: thread (phase, j) of the first PH
// phases (32, or 8 for a head with few records) owns dims 4j..4j+3 of chunks
// phase, phase + PH, ...; it loads 8 of its chunk records at once (so every
// load of a pass is in flight together), then folds them in with a running
// maximum.  The PH phases are combined through LDS.  When idx is requested
// the block then assembles the ascending sampled-index list from the chunks'
// union entries.
constexpr int MERGE_PH = 32;  // chunk phases per head (x 32 threads of 4 dims = 1024 threads)
constexpr int MERGE_CPT = 8;  // chunks a thread loads before combining them
// A head with at most MERGE_PH_FEW * MERGE_CPT records is merged in
// MERGE_PH_FEW phases (one pass of loads each): fewer waves per block, so a
// grid of many small heads is resident at once.  Both merges pick the phase
// count the same way, so they fold the records in the same order.
constexpr int MERGE_PH_FEW = 8;
__host__ __device__ constexpr int merge_phases(int64_t nrec) {
  return nrec <= (int64_t)MERGE_PH_FEW * MERGE_CPT ? MERGE_PH_FEW : MERGE_PH;
}

// One thread's share of a head's merge: records ph, ph + PH, ... of
// nrec at p0 (record stride cs), dims d0 .. d0 + 3.  Record r is chunk r's,
// or, when the sampling blocks took the bitmap chunks `span` at a time,
// chunk r * span for r < nsp and chunk nlt + r - nsp after.  A pass loads
// MERGE_CPT records at once (independent loads; records past the last
// re-read the last one and are dropped, or with few phases are not read),
// then folds them in with a running maximum (rescaled sums).  The records'
// counts are summed when `counts` is set.
struct MergePart {
  float m, l;
  f32x4 o;
  int cnt;
};
template <int PH>
__device__ inline MergePart merge_fold(const float *__restrict__ p0, int64_t cs, int64_t nrec, int ph, int d0,
                                       bool counts, int64_t nsp = 0, int span = 1, int64_t nlt = 0) {
  MergePart r{-INFINITY, 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}, 0};
  for (int64_t c0 = ph; c0 < nrec; c0 += (int64_t)PH * MERGE_CPT) {
    f32x2 ml[MERGE_CPT];
    int cn[MERGE_CPT];
    f32x4 oc[MERGE_CPT];
    auto load = [&](int k) {
      const int64_t ri = min(c0 + (int64_t)k * PH, nrec - 1);
      const int64_t ci = ri < nsp ? ri * span : nlt + ri - nsp;
      const float *rec = p0 + ci * cs;
      ml[k] = *(const f32x2 *)rec;  // m, l
      cn[k] = counts ? __builtin_bit_cast(int, rec[2]) : 0;
      oc[k] = *(const f32x4 *)(rec + 4 + d0);
    };
    // with few phases (one pass), the loads the wave's first phase (lane 0's,
    // the lowest) has no record for are skipped wave-wide; with many, every
    // load is issued (measured: the skips' branches cost more there)
    if constexpr (PH == MERGE_PH) {
#pragma unroll
      for (int k = 0; k < MERGE_CPT; ++k) load(k);
    } else {
      const int64_t cw = (int64_t)__builtin_amdgcn_readfirstlane((int)c0);
#pragma unroll
      for (int k = 0; k < MERGE_CPT; ++k) {
        ml[k] = f32x2{-INFINITY, 0.0f};
        cn[k] = 0;
        oc[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (cw + (int64_t)k * PH < nrec) load(k);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the pass is issued before any result is used
    // branch-free fold (a branch would let the compiler sink the loads into
    // it, one round trip each); an empty side gets weight 0
#pragma unroll
    for (int k = 0; k < MERGE_CPT; ++k) {
      const bool live = c0 + (int64_t)k * PH < nrec;
      const float mc = live ? ml[k][0] : -INFINITY;
      const float mn = fmaxf(r.m, mc);
      const float a = r.m > -INFINITY ? __expf(r.m - mn) : 0.0f;
      const float bsc = mc > -INFINITY ? __expf(mc - mn) : 0.0f;
      r.l = r.l * a + ml[k][1] * bsc;
      // an empty record's o need not have been written (m = -inf, l = 0)
      r.o = bsc > 0.0f ? r.o * a + oc[k] * bsc : r.o * a;
      r.m = mn;
      r.cnt += live ? cn[k] : 0;
    }
  }
  return r;
}

// The PH phases' states (in LDS) folded in phase order for the 4 dims
// of slot s: writes out[0..3], and the log-sum-exp and count when asked.
template <int NS, int PH>
__device__ inline void merge_finish(const f32x4 (&red_o)[PH][NS], const float (&red_m)[PH],
                                    const float (&red_l)[PH], const int (&red_c)[PH], int s,
                                    float *__restrict__ out, float *lse, int32_t *count) {
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < PH; ++p) M = fmaxf(M, red_m[p]);
  f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
  float ls = 0.0f;
  int cs_ = 0;
#pragma unroll
  for (int p = 0; p < PH; ++p) {
    const float sc = red_m[p] > -INFINITY ? __expf(red_m[p] - M) : 0.0f;
    o += red_o[p][s] * sc;
    ls += red_l[p] * sc;
    cs_ += red_c[p];
  }
  const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
  *(f32x4 *)out = o * inv;
  if (lse) *lse = ls > 0.0f ? M + logf(ls) : -INFINITY;
  if (count) *count = cs_;
}

template <int PH>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4, 4))) void merge_kernel(const float *__restrict__ part, int Hq, int Hkv, int G,
                                                     int64_t nchunks, int64_t chunk, float *__restrict__ out,
                                                     float *__restrict__ lse, int32_t *__restrict__ count,
                                                     int32_t *__restrict__ idx, int64_t cap,
                                                     const uint32_t *__restrict__ ent,
                                                     const int32_t *__restrict__ ent_cnt, int64_t nlt, int span) {
  __shared__ f32x4 red_o[PH][32];
  __shared__ float red_m[PH], red_l[PH];
  __shared__ int red_c[PH];
  __shared__ int wsum[16];
  // unit-minor order, as the sampling kernel's grid: block i serves unit
  // i % U, so it runs on the same XCD as the blocks that wrote its partials
  touch_kernargs<2>();  // 112 bytes of arguments
  // (32-bit index arithmetic: a 64-bit division is a long instruction chain)
  const uint32_t U32 = gridDim.x / (uint32_t)G, bx = blockIdx.x;
  const int64_t u = (int64_t)(bx % U32);
  const int hg = (int)(bx / U32);
  const int b = (int)u / Hkv;
  const int h = ((int)u % Hkv) * G + hg;
  const int64_t bh = (int64_t)b * Hq + h;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float *p0 = part + (u * nchunks * G + hg) * PSTRIDE;
  const int64_t cs = (int64_t)G * PSTRIDE;

  // thread (phase, j) of the first PH phases: dims 4j..4j+3 of records
  // phase, phase + PH, ... (the records the sampling blocks filled, in the
  // same order as the merge without index lists, so that both give the same
  // bits)
  const int ph = t >> 5, j = t & 31;
  const int64_t nsp = (nlt + span - 1) / span;  // records of the bitmap chunks
  if (ph < PH) {
    const MergePart mpart = merge_fold<PH>(p0, cs, nsp + nchunks - nlt, ph, 4 * j, true, nsp, span, nlt);
    red_o[ph][j] = mpart.o;
    if (j == 0) {
      red_m[ph] = mpart.m;
      red_l[ph] = mpart.l;
      red_c[ph] = mpart.cnt;
    }
  }
  __syncthreads();
  if (t < 32)
    merge_finish<32, PH>(red_o, red_m, red_l, red_c, t, out + bh * D + 4 * t, t == 0 && lse ? lse + bh : nullptr,
                     t == 0 && count ? count + bh : nullptr);
  if (!idx) return;
  // Index list: chunk c's keys of this head start at the sum of the earlier
  // chunks' counts (their partial records hold them).  Chunks are taken 1024
  // at a time: one exclusive scan of their counts, then each wave copies whole
  // chunks (ballot + prefix count over the union entries, which are in key
  // order within a chunk).
  __shared__ int coff[1024];
  int32_t *dst = idx + bh * cap;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  for (int64_t g0 = 0; g0 < nchunks; g0 += 1024) {
    const int64_t ci = g0 + t;
    const int c = ci < nchunks ? max(__builtin_bit_cast(int, p0[ci * cs + 2]), 0) : 0;
    int incl = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();  // wsum / coff of the previous group no longer read
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      wpre += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
    coff[t] = base + wpre + incl - c;
    base += tot;
    __syncthreads();
    const int ng = (int)min((int64_t)1024, nchunks - g0);
    for (int k = wave; k < ng; k += 16) {
      const int64_t cc = g0 + k;
      // clamp: stays inside the workspace even if the entries were not written
      // (a sampling block that took several tiles keeps their entries in
      // its first tile's region and the ones after it)
      const int ne = (int)min((int64_t)max(ent_cnt[u * nchunks + cc], 0), (nchunks - cc) * 2 * chunk);
      const uint32_t *src = ent + (u * nchunks + cc) * (2 * chunk);
      int o = coff[k];
      for (int e0 = 0; e0 < ne; e0 += 64) {
        const int e = e0 + lane;
        uint32_t v = 0;
        bool f = false;
        if (e < ne) {
          v = src[e];
          f = (v >> (16 + hg)) & 1u;
        }
        const uint64_t bal = __ballot(f);
        const int pre = __popcll(bal & lt);
        if (f && o + pre < cap) dst[o + pre] = (int32_t)(cc * chunk + (v & 0xffffu));
        o += __popcll(bal);
      }
    }
  }
}

// --------------------------------------------------------------------------
// The same merge without the index list (up to four heads per unit),
// spread four times wider: one block
// of 256 threads per (query head, quarter of the output dims), so that a
// head's partial records are read by four compute units.  Thread (phase,
// j) owns dims 32 q + 4 j .. + 3 of records phase, phase + PH, ...; each
// block reads every record's m and l, the first quarter also its count.
// With span > 1 only the records the sampling blocks filled are read (one per
// block: chunks 0, span, 2 span, ... below nlt, every chunk from nlt on).

template <int PH>
__global__ __launch_bounds__(256) void merge_q_kernel(const float *__restrict__ part, int Hq, int Hkv, int G,
                                                      int64_t nchunks, int64_t nlt, int span,
                                                      float *__restrict__ out, float *__restrict__ lse,
                                                      int32_t *__restrict__ count) {
  __shared__ f32x4 red_o[PH][8];
  __shared__ float red_m[PH], red_l[PH];
  __shared__ int red_c[PH];
  touch_kernargs<1>();  // 64 bytes of arguments
  // unit-minor order, as the sampling kernel's grid: block i serves unit
  // i % U, so it runs on the XCD of the blocks that wrote its partials
  // (32-bit index arithmetic: a 64-bit division is a long instruction chain)
  const uint32_t U32 = gridDim.x / (4u * (uint32_t)G), bx = blockIdx.x;
  const int64_t u = (int64_t)(bx % U32);
  const uint32_t rest = bx / U32;
  const int hg = (int)(rest % (uint32_t)G), qq = (int)(rest / (uint32_t)G);
  const int b = (int)u / Hkv;
  const int h = ((int)u % Hkv) * G + hg;
  const int64_t bh = (int64_t)b * Hq + h;
  const int t = threadIdx.x;
  const float *p0 = part + (u * nchunks * G + hg) * PSTRIDE;
  const int64_t cs = (int64_t)G * PSTRIDE;
  const int ph = t >> 3, j = t & 7;
  const bool counts = qq == 0;  // the first quarter also writes the log-sum-exp and the count
  const int64_t nsp = (nlt + span - 1) / span;  // records of the bitmap chunks
  const MergePart mpart = merge_fold<PH>(p0, cs, nsp + nchunks - nlt, ph, 32 * qq + 4 * j, counts, nsp, span, nlt);
  red_o[ph][j] = mpart.o;
  if (j == 0) {
    red_m[ph] = mpart.m;
    red_l[ph] = mpart.l;
    red_c[ph] = mpart.cnt;
  }
  __syncthreads();
  if (t < 8)
    merge_finish<8, PH>(red_o, red_m, red_l, red_c, t, out + bh * D + 32 * qq + 4 * t,
                    t == 0 && counts && lse ? lse + bh : nullptr, t == 0 && counts && count ? count + bh : nullptr);
}

hipError_t launch_merge(int B, int Hq, int Hkv, int64_t n, int L, const DecodeGeom &geo, const DecodeWs &ws,
                        float *out, float *lse, int32_t *idx, int64_t cap, int32_t *count, hipStream_t s,
                        int64_t nlt, int span) {
  (void)n;
  (void)L;
  const int G = Hq / Hkv;
  // the wider merge pays with up to four heads per unit (measured: 96K
  // 4.96 -> 3.9 us, one head per unit 13.9 -> 10.5 us) but not with eight
  // (5.3 -> 6.4 us)
  const int64_t nl = span > 1 ? nlt : 0;
  const int sp = span > 1 ? span : 1;
  const int64_t nrec = (nl + sp - 1) / sp + geo.nchunks - nl;  // records per head
  const bool few = merge_phases(nrec) == MERGE_PH_FEW;
  if (!idx && G <= 4) {
    // a block of PH * 8 threads per (head, quarter of the dims)
    const dim3 grid((unsigned)(4 * (int64_t)B * Hq));
    if (few)
      merge_q_kernel<MERGE_PH_FEW><<<grid, MERGE_PH_FEW * 8, 0, s>>>(ws.part, Hq, Hkv, G, geo.nchunks, nl, sp, out,
                                                                      lse, count);
    else
      merge_q_kernel<MERGE_PH><<<grid, MERGE_PH * 8, 0, s>>>(ws.part, Hq, Hkv, G, geo.nchunks, nl, sp, out, lse,
                                                              count);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((int64_t)B * Hq));
  if (few)
    merge_kernel<MERGE_PH_FEW><<<grid, 1024, 0, s>>>(ws.part, Hq, Hkv, G, geo.nchunks, geo.chunk, out, lse, count,
                                                     idx, cap, ws.ent, ws.ent_cnt, nl, sp);
  else
    merge_kernel<MERGE_PH><<<grid, 1024, 0, s>>>(ws.part, Hq, Hkv, G, geo.nchunks, geo.chunk, out, lse, count, idx,
                                                 cap, ws.ent, ws.ent_cnt, nl, sp);
  return hipGetLastError();
}

}  // namespace mp
