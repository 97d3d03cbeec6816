// Bucketed hash tables of MagicPIG (arXiv 2410.16179v2): each of the L
// SimHash tables maps a K-bit code to the keys that carry it (Section 2.2
// "Locality sensitive hashing": L hash tables of K-bit codes; Section 4.4,
// the retrieval step that looks the query's L codes up in pre-built
// tables).  Here the tables are built on the GPU from the code store and kept
// in HBM; a decode reads only the query's buckets, counts every key's
// collisions in LDS and writes the union lists of the keys that collide in
// at least two tables -- the same sets as the full collision scan, since a
// key sits in the query's bucket of table l exactly when its code of table l
// equals the query's.
#include <hip/hip_ext.h>

#include "mp_internal.h"

namespace mp {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

BucketLayout bucket_layout(void *base, int64_t U, int64_t cap, int K, int L) {
  BucketLayout b;
  b.nbins = 1 << K;
  b.bchunks = (cap + BK_R - 1) / BK_R;
  const size_t off_bytes = align256(sizeof(uint32_t) * (size_t)U * L * b.nbins * b.bchunks);
  b.off = (uint32_t *)base;  // a NULL base asks for the size only
  b.keys = base ? (uint16_t *)((char *)base + off_bytes) : nullptr;
  b.bytes = off_bytes + align256(sizeof(uint16_t) * (size_t)U * L * cap);
  return b;
}

// Exclusive prefix sum over the 256 threads of a block (wave scans, then the
// four wave totals through LDS); *total receives the sum.  Every thread of the
// block must call it.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t *wsum, uint32_t *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    pre += w < wave ? wsum[w] : 0u;
    tot += wsum[w];
  }
  __syncthreads();  // wsum may be reused by the caller
  *total = tot;
  return pre + incl - v;
}

// --------------------------------------------------------------------------
// Build: one block per (unit, table, chunk).  Counting sort of the chunk's
// keys by code: a histogram of the 2^K codes in LDS (16-bit counters, two
// per word), its exclusive prefix sum gives the bucket starts, and each key
// takes the next slot of its bucket (an LDS atomic: the order of equal codes
// inside a bucket is not fixed, which the lookup does not depend on).
constexpr int BB_KPT = BK_R / 256;  // keys per thread

__global__ __launch_bounds__(256) void bucket_build_kernel(const uint16_t *__restrict__ codes, int64_t cap, int K,
                                                           int64_t c0, int64_t nc, int64_t n1, int64_t bchunks,
                                                           uint32_t *__restrict__ boff,
                                                           uint16_t *__restrict__ bkeys) {
  extern __shared__ uint32_t hist[];  // 2^K 16-bit counters, two per word
  __shared__ uint32_t wsum[4];
  const int nbins = 1 << K;
  const int nw = nbins >> 1;  // K >= 1
  const int64_t ci = c0 + (int64_t)blockIdx.x % nc;
  const int64_t ul = (int64_t)blockIdx.x / nc;  // unit * L + table
  const int64_t r0 = ci * BK_R;
  const int nk = (int)(min(r0 + BK_R, n1) - r0);
  const uint16_t *src = codes + ul * cap + r0;
  for (int i = threadIdx.x; i < nw; i += 256) hist[i] = 0u;
  uint32_t cd[BB_KPT];
#pragma unroll
  for (int k = 0; k < BB_KPT; ++k) {
    const int j = threadIdx.x + 256 * k;
    cd[k] = src[j < nk ? j : 0];  // every load in flight; keys past the chunk's last are not counted
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < BB_KPT; ++k)
    if ((int)threadIdx.x + 256 * k < nk) atomicAdd(&hist[cd[k] >> 1], 1u << (16 * (cd[k] & 1u)));
  __syncthreads();
  // thread t owns counter words [t * wpt, (t + 1) * wpt): bins 2 t wpt ..
  const int wpt = nw > 256 ? nw / 256 : 1;
  const int w0 = threadIdx.x * wpt;
  const bool owns = w0 < nw;
  uint32_t sum = 0;
  if (owns)
    for (int w = 0; w < wpt; ++w) sum += (hist[w0 + w] & 0xffffu) + (hist[w0 + w] >> 16);
  uint32_t total;
  uint32_t run = block_excl_scan(sum, wsum, &total);
  uint32_t *off = boff + ul * (int64_t)nbins * bchunks + ci;  // bucket c's word at off[c * bchunks]
  if (owns) {
    for (int w = 0; w < wpt; ++w) {
      const uint32_t h = hist[w0 + w];
      const uint32_t a = run, b = run + (h & 0xffffu);
      off[(int64_t)(2 * (w0 + w)) * bchunks] = a | ((h & 0xffffu) << 16);
      off[(int64_t)(2 * (w0 + w) + 1) * bchunks] = b | ((h >> 16) << 16);
      hist[w0 + w] = a | (b << 16);  // the buckets' next free slots
      run = b + (h >> 16);
    }
  }
  __syncthreads();
  uint16_t *dst = bkeys + ul * cap + r0;
#pragma unroll
  for (int k = 0; k < BB_KPT; ++k) {
    const int j = threadIdx.x + 256 * k;
    if (j < nk) {
      const uint32_t sh = 16 * (cd[k] & 1u);
      const uint32_t old = atomicAdd(&hist[cd[k] >> 1], 1u << sh);
      dst[(old >> sh) & 0xffffu] = (uint16_t)j;
    }
  }
}

hipError_t launch_bucket_build(const uint16_t *codes, int64_t U, int64_t cap, int K, int L, int64_t n0, int64_t n1,
                               const BucketLayout &bl, hipStream_t s) {
  const int64_t c0 = n0 / BK_R, c1 = (n1 + BK_R - 1) / BK_R;
  const int64_t nc = c1 - c0;
  if (nc <= 0 || U <= 0) return hipSuccess;
  const size_t lds = sizeof(uint32_t) * (size_t)(bl.nbins / 2);
  bucket_build_kernel<<<dim3((unsigned)(U * L * nc)), 256, lds, s>>>(codes, cap, K, c0, nc, n1, bl.bchunks, bl.off,
                                                                     bl.keys);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// Lookup (per decode step): one block per (unit, query head, chunk of BK_R
// keys below nb).
//  1. Segments: for table l the query's bucket c = qcode[l] holds the
//     entries start .. start + count - 1 of the chunk's table l (one word).
//     Thread t reads the words of tables t * spt .. (all loads in flight),
//     and a block-wide prefix sum of the counts numbers the entries.
//  2. Entries, in windows of BL_W: each thread writes its own segments'
//     table number into an LDS slot per entry of the window, then thread t
//     takes entries t, t + 256, ... of the window (all key loads in flight)
//     and records each collision in the head's LDS bitmaps: "seen in one
//     table" and, when already seen, "seen in two" (an atomic OR returns the
//     old word; a thread's ORs of a window are all issued before it reads
//     any old word).
//  3. The "seen in two tables" bitmap of the chunk is written to the head's
//     bitmap in the workspace; the sampling kernel compacts it per tile.
constexpr int BL_W = 2048;       // entries per window
constexpr int BL_EPT = BL_W / 256;  // entries per thread and window
constexpr int BL_WORDS = BK_R / 32;

__global__ __launch_bounds__(256) void bucket_lookup_kernel(const uint16_t *__restrict__ qcodes,
                                                            const uint32_t *__restrict__ boff,
                                                            const uint16_t *__restrict__ bkeys, int Hq, int Hkv, int G,
                                                            int64_t nb, int64_t cap, int K, int L, int64_t bchunks,
                                                            int64_t nbc, int64_t bwords, uint32_t *__restrict__ sbits) {
  __shared__ uint32_t seen1[BL_WORDS], seen2[BL_WORDS];
  __shared__ uint32_t segbeg[MAX_L + 1], segsrc[MAX_L];
  __shared__ uint16_t eseg[BL_W];
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x;
  touch_kernargs<2>();  // 96 bytes of arguments
  // unit-minor order, as the sampling grid: block i serves unit i % U, so
  // (with U a multiple of the 8 XCDs) it runs on the XCD whose blocks read
  // its words; then head, then chunk
  // (32-bit index arithmetic: a 64-bit division is a long instruction chain)
  const uint32_t U32 = gridDim.x / ((uint32_t)nbc * (uint32_t)G), bx = blockIdx.x;
  const int ui = (int)(bx % U32);
  const uint32_t hc = bx / U32;
  const int h = (int)(hc % (uint32_t)G);
  const int64_t ci = (int64_t)(hc / (uint32_t)G);
  const int64_t u = ui;
  const int64_t ug = u * G + h;  // unit * G + head
  const int64_t qrow = (int64_t)(ui / Hkv) * Hq + (int64_t)(ui % Hkv) * G + h;
  const int64_t r0 = ci * BK_R, r1 = min(r0 + BK_R, nb);
  const int nbins = 1 << K;
  for (int i = tid; i < BL_WORDS; i += 256) {
    seen1[i] = 0u;
    seen2[i] = 0u;
  }
  // ---- 1. segments: thread t owns tables [t * spt, t * spt + spt)
  constexpr int MAX_SPT = (MAX_L + 255) / 256;
  const int spt = (L + 255) / 256;
  const int l0 = tid * spt;
  uint32_t len[MAX_SPT], src[MAX_SPT];
  {
    uint32_t qc[MAX_SPT];
#pragma unroll
    for (int k = 0; k < MAX_SPT; ++k) qc[k] = k < spt ? qcodes[qrow * L + min(l0 + k, L - 1)] : 0u;
#pragma unroll
    for (int k = 0; k < MAX_SPT; ++k) {
      const int l = min(l0 + k, L - 1);
      const uint32_t wv = k < spt ? boff[((u * L + l) * nbins + qc[k]) * bchunks + ci] : 0u;
      const bool mine = k < spt && l0 + k < L;
      src[k] = wv & 0xffffu;
      len[k] = mine ? wv >> 16 : 0u;
    }
  }
  uint32_t part = 0;
#pragma unroll
  for (int k = 0; k < MAX_SPT; ++k) part += len[k];
  uint32_t total;
  uint32_t run = block_excl_scan(part, wsum, &total);
#pragma unroll
  for (int k = 0; k < MAX_SPT; ++k) {
    if (k < spt && l0 + k < L) {
      segbeg[l0 + k] = run;
      segsrc[l0 + k] = src[k];
      run += len[k];
    }
  }
  if (tid == 0) segbeg[L] = total;
  __syncthreads();
  // ---- 2. entries, window by window
  const uint16_t *kbase = bkeys + u * (int64_t)L * cap + r0;
  for (uint32_t w0 = 0; w0 < total; w0 += BL_W) {
    const uint32_t w1 = min(total, w0 + (uint32_t)BL_W);
#pragma unroll
    for (int k = 0; k < MAX_SPT; ++k) {
      if (k < spt && l0 + k < L) {
        const uint32_t b = max(segbeg[l0 + k], w0), e = min(segbeg[l0 + k + 1], w1);
        for (uint32_t x = b; x < e; ++x) eseg[x - w0] = (uint16_t)(l0 + k);
      }
    }
    __syncthreads();
    uint32_t key[BL_EPT];
#pragma unroll
    for (int k = 0; k < BL_EPT; ++k) {
      const uint32_t e = min(w0 + (uint32_t)tid + 256u * k, w1 - 1u);
      const int l = eseg[e - w0];
      key[k] = kbase[(int64_t)l * cap + segsrc[l] + (e - segbeg[l])];
    }
    // every atomic OR of the window goes out before any old word is looked
    // at (one LDS round trip instead of one per entry); slots past the
    // window issue none (they would all hit the window's last key's word)
    uint32_t bit[BL_EPT], old[BL_EPT];
#pragma unroll
    for (int k = 0; k < BL_EPT; ++k) {
      bit[k] = 1u << (key[k] & 31u);
      old[k] = 0u;
      if (w0 + (uint32_t)tid + 256u * k < w1) old[k] = atomicOr(&seen1[key[k] >> 5], bit[k]);
    }
#pragma unroll
    for (int k = 0; k < BL_EPT; ++k)
      if (old[k] & bit[k]) atomicOr(&seen2[key[k] >> 5], bit[k]);
    __syncthreads();  // the window's slots are rewritten next
  }
  __syncthreads();
  // ---- 3. the chunk's "two tables" words into the head's bitmap
  const int nw = (int)((r1 - r0) / 32);
  uint32_t *dst = sbits + ug * bwords + r0 / 32;
  for (int i = tid; i < nw; i += 256) dst[i] = seen2[i];
}

hipError_t launch_bucket_lookup(const uint16_t *qcodes, const BucketLayout &bl, int B, int Hq, int Hkv, int64_t n,
                                int64_t nb, int64_t cap, int K, int L, int64_t nsh, int64_t nst, const DecodeGeom &geo,
                                const DecodeWs &ws, hipStream_t s, hipEvent_t ev_start) {
  (void)B;
  (void)n;
  (void)nsh;
  (void)nst;
  const int G = Hq / Hkv;
  const int64_t nbc = (nb + BK_R - 1) / BK_R;
  if (nbc <= 0) return hipSuccess;
  const dim3 grid((unsigned)(geo.U * G * nbc));
  hipExtLaunchKernelGGL(bucket_lookup_kernel, grid, dim3(256), 0, s, ev_start, nullptr, 0, qcodes, bl.off, bl.keys,
                        Hq, Hkv, G, nb, cap, K, L, bl.bchunks, nbc, geo.nchunks_max * (SCAN_TILE / 32), ws.bits);
  return hipGetLastError();
}

}  // namespace mp
