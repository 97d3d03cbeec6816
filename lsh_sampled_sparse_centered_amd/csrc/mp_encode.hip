// SimHash encoder of MagicPIG (arXiv 2410.16179v2): key mean, projection
// packing and the bf16 matrix-core projection + sign packing that produces
// the table-major code store (Section 2.2 "Locality sensitive hashing";
// Section 4.3 "Hash function selection" and "Data pre-processing").
#include <algorithm>
#include <type_traits>

#include "mp_internal.h"

namespace mp {

// ---------------------------------------------------------------------------
// Projection packing: W[d][K*L] fp32 -> negated bf16 tiles in matrix-core
// A-operand order.  Element e of lane l in k-step s of tile t is
//   -W[16 s + 8 (l / 32) + e][K (t tpt + j) + b],  K j + b = enc_row_col(l % 32),
// and 0 where j >= tpt or t tpt + j >= L.  The tiles hold -bf16(W) (negation
// is exact and commutes with rounding), so the encoders' accumulators hold
// -z for each projection z and the sign bit of an accumulator is (z > 0)
// directly (see sign_bits16).
// One thread per (tile, k-step, lane) writes 16 bytes.
__global__ void proj_pack_kernel(const float *__restrict__ W, int K, int L, int ntiles, uint4 *__restrict__ Wp) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)ntiles * KSTEPS * 64) return;
  const int lane = (int)(gid & 63);
  const int s = (int)((gid >> 6) % KSTEPS);
  const int t = (int)(gid / (64 * KSTEPS));
  const int tpt = enc_tpt(K);
  const int p = enc_row_col(lane & 31);  // bit of the tile's word
  const int j = p / K, b = p % K, l = t * tpt + j;
  const bool live = j < tpt && l < L;
  const int col = l * K + b;
  const int ncol = K * L;
  const int d0 = 16 * s + 8 * (lane >> 5);
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (__bf16)(live ? -W[(int64_t)(d0 + e) * ncol + col] : 0.0f);
  Wp[gid] = __builtin_bit_cast(uint4, v);
}

hipError_t launch_proj_pack(const float *W, int K, int L, void *Wp, hipStream_t s) {
  const int ntiles = enc_ntiles(K, L);
  const int64_t total = (int64_t)ntiles * KSTEPS * 64;
  if (total == 0) return hipSuccess;
  proj_pack_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s>>>(W, K, L, ntiles, (uint4 *)Wp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Key mean k_avg = (1/n) sum_i k_i per unit, accumulated in fp64 and rounded
// once to fp32.  Stage 1: each block sums KM_ROWS rows of one unit
// (16 lanes x 8 dims cover a row; 16 x KM_UNR rows in flight per pass, all
// loads of a pass issued together).
// Stage 2: one block per unit adds the stage-1 sums in a fixed order
// (deterministic).
constexpr int KM_ROWS = 512;   // rows per block
constexpr int KM_UNR = 8;      // rows a 16-lane group has in flight
constexpr int KM_SLICES = 8;   // threads per dimension in the final sum

int kmean_parts(int64_t n) { return (int)((n + KM_ROWS - 1) / KM_ROWS); }

template <typename T>
__device__ inline void load8(const T *p, float (&v)[8]);
template <>
__device__ inline void load8<float>(const float *p, float (&v)[8]) {
  const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[e + 4] = b[e]; }
}
template <>
__device__ inline void load8<__bf16>(const __bf16 *p, float (&v)[8]) {
  const bf16x8 a = *(const bf16x8 *)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
}

// A row slice of 8 elements as raw 16-byte words (so the loads can all be
// issued before any is converted).
template <typename T>
struct KRow;
template <>
struct KRow<__bf16> {
  uint4 a;
  __device__ void load(const __bf16 *p) { a = *(const uint4 *)p; }
  __device__ void add_to(double (&acc)[8], bool live) const {
    const bf16x8 b = __builtin_bit_cast(bf16x8, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += live ? (double)(float)b[e] : 0.0;
  }
};
template <>
struct KRow<float> {
  uint4 a, b;
  __device__ void load(const float *p) {
    a = *(const uint4 *)p;
    b = *(const uint4 *)(p + 4);
  }
  __device__ void add_to(double (&acc)[8], bool live) const {
    const f32x4 x = __builtin_bit_cast(f32x4, a), y = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] += live ? (double)x[e] : 0.0;
      acc[e + 4] += live ? (double)y[e] : 0.0;
    }
  }
};

template <typename T>
__global__ __launch_bounds__(256) void kmean_partial_kernel(const T *__restrict__ Kc, int64_t n, int64_t cap,
                                                            int nparts, double *__restrict__ partial) {
  __shared__ double red[16][D];
  const int64_t u = blockIdx.y;
  const int p = blockIdx.x;
  const int j16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;
  const int64_t r0 = (int64_t)p * KM_ROWS, r1 = min(n, r0 + KM_ROWS);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const T *base = Kc + u * cap * D + 8 * j16;
  for (int64_t r = r0 + rsub; r < r1; r += 16 * KM_UNR) {
    // every load of the pass is issued before any is used: rows past the
    // block's last re-read its last row and add nothing
    KRow<T> v[KM_UNR];
#pragma unroll
    for (int k = 0; k < KM_UNR; ++k) v[k].load(base + min(r + 16 * k, r1 - 1) * D);
    __builtin_amdgcn_sched_barrier(0);  // keeps the loads ahead of every use
#pragma unroll
    for (int k = 0; k < KM_UNR; ++k) v[k].add_to(acc, r + 16 * k < r1);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub][8 * j16 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += red[r][threadIdx.x];
    partial[(u * nparts + p) * D + threadIdx.x] = s;
  }
}

__global__ __launch_bounds__(D * KM_SLICES) void kmean_final_kernel(const double *__restrict__ partial, int nparts,
                                                                   int64_t n, float *__restrict__ kmean) {
  // thread (slice, dim) adds parts slice, slice + KM_SLICES, ... (eight
  // loads in flight: unconditional, parts past the last re-read it and add
  // nothing), then the slices are added in slice order: a fixed order
  __shared__ double red[KM_SLICES][D];
  const int64_t u = blockIdx.x;
  const int dim = threadIdx.x % D, slice = threadIdx.x / D;
  const double *p0 = partial + u * (int64_t)nparts * D + dim;
  double s8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int p = slice; p < nparts; p += 8 * KM_SLICES) {
    double v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p0[(int64_t)min(p + k * KM_SLICES, nparts - 1) * D];
    __builtin_amdgcn_sched_barrier(0);  // keeps the loads ahead of every use
#pragma unroll
    for (int k = 0; k < 8; ++k) s8[k] += p + k * KM_SLICES < nparts ? v[k] : 0.0;
  }
  red[slice][dim] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
  __syncthreads();
  if (slice == 0) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < KM_SLICES; ++k) s += red[k][dim];
    kmean[u * D + dim] = (float)(s / (double)n);
  }
}

hipError_t launch_kmean(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, double *partial,
                        int nparts, float *kmean, hipStream_t s) {
  dim3 g1((unsigned)nparts, (unsigned)U);
  if (kv_dtype == 0)
    kmean_partial_kernel<__bf16><<<g1, 256, 0, s>>>((const __bf16 *)Kc, n, cap, nparts, partial);
  else
    kmean_partial_kernel<float><<<g1, 256, 0, s>>>((const float *)Kc, n, cap, nparts, partial);
  kmean_final_kernel<<<dim3((unsigned)U), D * KM_SLICES, 0, s>>>(partial, nparts, n, kmean);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Lift of Section 4.2, Equation 8 (an option; the pages do not use it).  The
// projections' extra row W[d] is packed per tile in the order of the tile
// word's bits (bf16, 0 past the tile's tables), so a lane reads the 16 values
// of its accumulator elements contiguously.
__global__ void proj_pack_lift_kernel(const float *__restrict__ W, int K, int L, int ntiles,
                                      uint16_t *__restrict__ wlift) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= ntiles * 32) return;
  const int t = gid >> 5, p = gid & 31, tpt = enc_tpt(K);
  const int j = p / K, b = p % K, l = t * tpt + j;
  const bool live = j < tpt && l < L;
  const __bf16 v = (__bf16)(live ? W[(int64_t)D * K * L + l * K + b] : 0.0f);
  wlift[gid] = __builtin_bit_cast(uint16_t, v);
}

hipError_t launch_proj_pack_lift(const float *W, int K, int L, uint16_t *wlift, hipStream_t s) {
  const int ntiles = enc_ntiles(K, L);
  if (ntiles == 0) return hipSuccess;
  proj_pack_lift_kernel<<<dim3((unsigned)((ntiles * 32 + 255) / 256)), dim3(256), 0, s>>>(W, K, L, ntiles, wlift);
  return hipGetLastError();
}

// Lift radius: the largest |x_i|^2 of x_i = bf16(fp32(k_i) - mu) per 512-row
// block (16 lanes per row, fp64), then per unit the largest block value, its
// square root rounded once to fp32.
template <typename T>
__global__ __launch_bounds__(256) void lift_partial_kernel(const T *__restrict__ Kc, int64_t n, int64_t cap,
                                                           const float *__restrict__ kmean, int nparts,
                                                           double *__restrict__ partial) {
  __shared__ double red[16];
  const int64_t u = blockIdx.y;
  const int p = blockIdx.x;
  const int j16 = threadIdx.x & 15, rsub = threadIdx.x >> 4;
  const int64_t r0 = (int64_t)p * KM_ROWS, r1 = min(n, r0 + KM_ROWS);
  float mv[8];
  load8<float>(kmean + u * D + 8 * j16, mv);
  double best = 0.0;
  for (int64_t r = r0 + rsub; r < r1; r += 16) {
    float v[8];
    load8<T>(Kc + (u * cap + r) * D + 8 * j16, v);
    double s2 = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = (double)(float)(__bf16)(v[e] - mv[e]);  // fp32 subtraction, bf16 rounding
      s2 += x * x;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s2 += __shfl_xor(s2, o);  // the row's 16 lanes
    best = fmax(best, s2);
  }
  if (j16 == 0) red[rsub] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    double m = 0.0;
    for (int k = 0; k < 16; ++k) m = fmax(m, red[k]);
    partial[u * nparts + p] = m;
  }
}

__global__ __launch_bounds__(256) void lift_final_kernel(const double *__restrict__ partial, int nparts,
                                                         float *__restrict__ rlift) {
  __shared__ double red[256];
  const int64_t u = blockIdx.x;
  double m = 0.0;
  for (int p = threadIdx.x; p < nparts; p += 256) m = fmax(m, partial[u * nparts + p]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) rlift[u] = (float)sqrt(red[0]);
}

hipError_t launch_lift_radius(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, const float *kmean,
                              double *partial, int nparts, float *rlift, hipStream_t s) {
  dim3 g1((unsigned)nparts, (unsigned)U);
  if (kv_dtype == 0)
    lift_partial_kernel<__bf16><<<g1, 256, 0, s>>>((const __bf16 *)Kc, n, cap, kmean, nparts, partial);
  else
    lift_partial_kernel<float><<<g1, 256, 0, s>>>((const float *)Kc, n, cap, kmean, nparts, partial);
  lift_final_kernel<<<dim3((unsigned)U), 256, 0, s>>>(partial, nparts, rlift);
  return hipGetLastError();
}

// The extra coordinate of lifted rows: with the row's B operands held by this
// lane (half of its dims) and its partner lane l ^ 32 (the other half),
// e = bf16(fp32(sqrt(max(0, r^2 - |x|^2)))) with |x|^2 summed in fp64.
__device__ inline float lift_coord(const bf16x8 (&xr)[KSTEPS], float r) {
  double s2 = 0.0;
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = (double)(float)xr[s][e];
      s2 += x * x;
    }
  s2 += __shfl_xor(s2, 32);
  const double rem = (double)r * (double)r - s2;
  return (float)(__bf16)(float)sqrt(rem > 0.0 ? rem : 0.0);
}

// Sign bits of lifted projections: the accumulator holds -z over the first d
// dims (negated tiles), the extra row W[d] is packed as is, and
// fl(-e w + (-z)) = -fl(z + e w) (one fp32 fma), so its sign bit is bit r =
// (z + e w > 0) as in sign_bits16 (an exact zero rounds to +0: bit 0).  wl
// holds the 16 bf16 extra-row values of this lane half's bits.
__device__ inline uint32_t sign_bits16_lift(const f32x16 &a, float e, const uint4 (&wl)[2]) {
  const bf16x8 w0 = __builtin_bit_cast(bf16x8, wl[0]), w1 = __builtin_bit_cast(bf16x8, wl[1]);
  uint32_t pos = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    const float w = r < 8 ? (float)w0[r & 7] : (float)w1[r & 7];
    const float nz = fmaf(-e, w, a[r]);
    pos = __builtin_amdgcn_alignbit(pos, __builtin_bit_cast(uint32_t, nz), 31u);
  }
  return pos & 0xffffu;
}

// ---------------------------------------------------------------------------
// Encoder.  Each block encodes ENC_ROWS rows of one unit for the tables
// [l0, l1) of its table group.  Wave w owns rows w*64 .. w*64+63 as two
// 32-row B operands held in registers (x = bf16(row - mu) for the 128 dims).
// Packed projection tiles are copied global -> LDS (double buffered, ENC_TG
// tiles per stage); per tile a wave issues 2 x 8 matrix-core ops (32x32x16
// bf16, fp32 accumulate).  Each accumulator's sign gives one bit (z > 0);
// the 16-bit masks of the two lane halves are swapped so that lane l holds
// the tile's 32-bit word of row w*64 + l, whose bit fields are the codes of
// the tile's tables, stored to out[u*out_su + l*out_sl + row*out_si].
//
// For appends the same pass copies the raw key row (and value row) into the
// cache when kcopy / vcopy are given.
template <typename T>
__device__ inline void load_row8(const T *p, float (&v)[8]) { load8<T>(p, v); }

template <typename T>
__device__ inline void store_row8(T *p, const float (&v)[8]);
template <>
__device__ inline void store_row8<float>(float *p, const float (&v)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int e = 0; e < 4; ++e) { a[e] = v[e]; b[e] = v[e + 4]; }
  *(f32x4 *)p = a;
  *(f32x4 *)(p + 4) = b;
}
template <>
__device__ inline void store_row8<__bf16>(__bf16 *p, const float (&v)[8]) {
  bf16x8 a;
#pragma unroll
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)v[e];  // exact: values came from bf16
  *(bf16x8 *)p = a;
}

// Bit r of the result is (z_r > 0) where the accumulator holds a[r] = -z_r
// (the packed tiles are negated, and the matrix core's products and sums
// are symmetric under negation): -z_r has its sign bit set exactly when
// z_r > 0.  An exactly zero projection -- a zero row, a zero projection
// column, or an exact cancellation -- accumulates to +0 from the +0 start
// (x + (-x) and +0 + (-0) round to +0), so it gives bit 0, as (z > 0) does.
// The sign bits are shifted in one per element (a funnel shift of (word,
// element) by 31, from element 15 down to 0).  Each element is copied to a
// scalar before the bit cast (a bit cast of the vector element itself has
// been compiled to a read of element 0 for every r).
__device__ inline uint32_t sign_bits16(const f32x16 &a) {
  uint32_t pos = 0;
#pragma unroll
  for (int r = 15; r >= 0; --r) {
    const float x = a[r];
    pos = __builtin_amdgcn_alignbit(pos, __float_as_uint(x), 31u);  // (pos << 1) | (z_r > 0)
  }
  return pos & 0xffffu;
}

// The kernel takes up to two independent row sets ("jobs", e.g. the keys to
// append and the queries of a decode step) and maps its linear block index
// onto (job, row block, unit, table group).
template <typename T, bool LIFT>
__global__ __launch_bounds__(64 * ENC_NW, MP_ENC_OCC) void encode_kernel(EncJob j0, EncJob j1, int njobs, const uint4 *__restrict__ wp,
                                                        int K, int L, const uint4 *__restrict__ wlift) {
  __shared__ uint4 wsh[2][ENC_TG * KSTEPS * 64];
  __shared__ uint16_t cst[ENC_NW][ENC_CST][64];  // a wave's codes of one stage, [table][row]
  const bool second = njobs > 1 && (int64_t)blockIdx.x >= j1.first_block;
  const EncJob &jb = second ? j1 : j0;
  const T *__restrict__ in = (const T *)jb.in;
  const int64_t in_su = jb.in_su, in_si = jb.in_si;
  const float *__restrict__ mu = jb.mu;
  const int64_t mu_su = jb.mu_su, mu_si = jb.mu_si, rows = jb.rows;
  uint16_t *__restrict__ out = jb.out;
  const int64_t out_su = jb.out_su, out_si = jb.out_si, out_sl = jb.out_sl;
  T *__restrict__ kcopy = (T *)jb.kcopy;
  const int64_t kc_su = jb.kc_su, kc_si = jb.kc_si;
  const T *__restrict__ vin = (const T *)jb.vin;
  T *__restrict__ vcopy = (T *)jb.vcopy;
  const int64_t local = (int64_t)blockIdx.x - jb.first_block;
  const int zt = (int)(local % jb.tsplit);
  const int64_t rest = local / jb.tsplit;
  const int64_t rb = rest % jb.rblocks;
  const int tables_per_block = jb.tpb;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int64_t u = rest / jb.rblocks;
  const int64_t row_w = rb * ENC_ROWS + wave * 64;  // first row of this wave
  const int l0 = zt * tables_per_block;
  const int l1 = min(L, l0 + tables_per_block);

  // tiles [t0, t1) hold tables [l0, l1) (l0 is a multiple of tpt)
  const int tpt = enc_tpt(K);
  const int t0 = K > 0 ? l0 / tpt : 0, t1 = K > 0 ? (l1 + tpt - 1) / tpt : 0;

  // Projection tiles [tg, tg + ENC_TG) are copied global -> LDS directly
  // (no registers): each wave moves whole 1 KB pieces, so the condition is
  // uniform per wave.  The barrier that ends a stage waits for them.
  constexpr int NT = 64 * ENC_NW;
#define MP_FETCH(buf_, tg_)                                                                        \
  do {                                                                                             \
    const int cnt_ = min(ENC_TG, t1 - (tg_)) * KSTEPS * 64;                                        \
    const uint4 *src_ = wp + (int64_t)(tg_)*KSTEPS * 64 + threadIdx.x;                             \
    _Pragma("unroll") for (int k_ = 0; k_ < (ENC_TG * KSTEPS * 64 + NT - 1) / NT; ++k_) {          \
      const int base_ = wave * 64 + k_ * NT;                                                       \
      if (base_ < cnt_)                                                                            \
        __builtin_amdgcn_global_load_lds((const void *)(src_ + k_ * NT),                           \
                                         (__attribute__((address_space(3))) void *)&wsh[buf_][base_], \
                                         16, 0, 0);                                                \
    }                                                                                              \
  } while (0)

  // the first stage's loads are issued before the rows are read, so the two
  // latencies overlap (this is what bounds small jobs)
  if (K > 0) MP_FETCH(0, t0);

  // appends: the table blocks of a row block copy the raw key and value rows
  // into the caches, each its share of the 16-byte pieces.  A thread's first
  // piece is loaded with the operand rows (one memory round trip for both)
  // and stored once they have arrived; further pieces (few blocks) follow.
  constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
  const int64_t cr0 = rb * ENC_ROWS;
  const int cnp = (kcopy && vcopy) ? (int)min((int64_t)ENC_ROWS, rows - cr0) * CPR : 0;  // pieces
  const int cfirst = zt * NT + (int)threadIdx.x, cstep = (int)jb.tsplit * NT;
  auto piece_src = [&](const T *base, int c) {
    return (const uint4 *)((const char *)(base + u * in_su + (cr0 + c / CPR) * in_si) + 16 * (c % CPR));
  };
  auto piece_dst = [&](T *base, int c) {
    return (uint4 *)((char *)(base + u * kc_su + (cr0 + c / CPR) * kc_si) + 16 * (c % CPR));
  };
  uint4 kx0 = {0u, 0u, 0u, 0u}, vx0 = {0u, 0u, 0u, 0u};
  if (cfirst < cnp) {
    kx0 = *piece_src(in, cfirst);
    vx0 = *piece_src(vin, cfirst);
  }

  // B operands: rows row_w + 32*nt + lane%32, dims 16 s + 8 half + e.  All
  // loads of a 32-row set are issued before any is used (one memory round
  // trip per set): rows past the end read the last row and are zeroed after.
  bf16x8 xb[2][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t r = row_w + 32 * nt + (lane & 31);
    const bool ok = r < rows;
    const int64_t rc = ok ? r : rows - 1;
    const T *rp = in + u * in_su + rc * in_si + 8 * half;
    float v[KSTEPS][8];
    if (mu) {  // the row and mean loads go out together
      const float *mp = mu + u * mu_su + rc * mu_si + 8 * half;
      float m[KSTEPS][8];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        load_row8<T>(rp + 16 * s, v[s]);
        load8<float>(mp + 16 * s, m[s]);
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[s][e] = v[s][e] - m[s][e];  // fp32 subtraction
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) load_row8<T>(rp + 16 * s, v[s]);
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[nt][s][e] = ok ? (__bf16)v[s][e] : (__bf16)0.0f;  // round to nearest even
  }
  // lifted rows: the extra coordinate of this lane's row of each set
  float ebar[2] = {0.0f, 0.0f};
  if constexpr (LIFT) {
    if (jb.rl) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int64_t r = min(row_w + 32 * nt + (lane & 31), rows - 1);
        ebar[nt] = lift_coord(xb[nt], jb.rl[u * jb.rl_su + r * jb.rl_si]);
      }
    }
  }

  if (cfirst < cnp) {
    *piece_dst(kcopy, cfirst) = kx0;
    *piece_dst(vcopy, cfirst) = vx0;
  }
  for (int c = cfirst + cstep; c < cnp; c += cstep) {  // both loads before both stores
    const uint4 kx = *piece_src(in, c), vx = *piece_src(vin, c);
    *piece_dst(kcopy, c) = kx;
    *piece_dst(vcopy, c) = vx;
  }

  const int64_t my_row = row_w + lane;  // row whose 32-bit words this lane assembles
  const bool my_ok = my_row < rows;
  uint16_t *my_out = out + u * out_su + my_row * out_si;

  if (K == 0) {
    for (int l = l0; l < l1; ++l)
      if (my_ok) my_out[(int64_t)l * out_sl] = 0;
    return;
  }

  __syncthreads();
  // A stage's sign words are cut into codes and stored at the start of the
  // next stage, so the stores complete while that stage's tiles run (the
  // wait for the next projection stage then does not wait for them).  Table
  // t*tpt + j of a tile is the bit field [K j, K j + K) of its word.
  uint32_t wd[ENC_TG];
  int tpend = 0, npend = 0;  // first tile and number of tiles pending
  // Key-major code rows (out_si = 1, the code store) with at most 8 tables
  // per tile go out as 16-byte stores of 8 rows of one table: the wave's
  // codes are transposed through LDS ([table][row]).  Each tile writes 8
  // slots without branches, in tile order, so the slots past a tile's tpt
  // codes are overwritten by the next tile's.  Otherwise each lane stores
  // its own 2-byte codes.
  const bool vec_out = out_si == 1 && tpt <= 8;
  auto emit_stage = [&]() {
    const int lb = tpend * tpt, le = min(l1, (tpend + npend) * tpt);
    if (vec_out) {
#pragma unroll
      for (int i = 0; i < ENC_TG; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          cst[wave][i * tpt + j][lane] = (uint16_t)__builtin_amdgcn_ubfe(wd[i], (uint32_t)(K * j), (uint32_t)K);
      const int nv = (le - lb) * 8;  // 16-byte pieces
      uint16_t *o = out + u * out_su + (int64_t)lb * out_sl + row_w;
#pragma unroll
      for (int k0 = 0; k0 < ENC_CST * 8; k0 += 64) {
        const int k = k0 + lane, t = k >> 3, g = k & 7;
        if (k < nv) {
          const uint4 v = *(const uint4 *)&cst[wave][t][8 * g];
          uint16_t *dst = o + (int64_t)t * out_sl + 8 * g;
          const int64_t r0 = row_w + 8 * g;
          if (r0 + 8 <= rows) {
            *(uint4 *)dst = v;
          } else {  // the unit's last rows: columns past them are not touched
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 8; ++e)
              if (r0 + e < rows) dst[e] = (uint16_t)(w4[e >> 1] >> (16 * (e & 1)));
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < ENC_TG; ++i)
        if (i < npend) {
          const int lt = (tpend + i) * tpt;
          uint16_t *o = my_out + (int64_t)lt * out_sl;
          for (int j = 0; j < min(tpt, l1 - lt); ++j)
            if (my_ok) o[(int64_t)j * out_sl] = (uint16_t)__builtin_amdgcn_ubfe(wd[i], (uint32_t)(K * j), (uint32_t)K);
        }
    }
  };
  // Fast path (2, 3 or 4 tables per tile, code region of the unit below
  // 2 GB): the next stage's projection copy is issued before this stage's
  // code stores, and a stage ends with a wait for all but the last
  // ENC_TG * TPT vector-memory operations (the code stores) and a barrier
  // without a memory fence, so no wave waits for its own code stores to be
  // written.  Each lane stores its row's codes directly (one 2-byte store per
  // table: a wave writes 128 contiguous bytes of a table row), and every lane
  // issues exactly ENC_TG * TPT stores per stage: codes of tables past l1,
  // of tiles past the stage's last and of rows past the end get an offset
  // past the buffer's end, which the hardware drops.  No LDS is written
  // between the copy's issue and the barrier.  The wait relies on the vector
  // memory counter retiring loads and stores in issue order, so "all but the
  // last NST" includes every projection-copy load issued before the stores.
  const int64_t oreach = 2 * ((int64_t)(L - 1) * out_sl + (rows - 1) * out_si + 1);  // bytes of the unit's codes
  const int ftpt = (oreach <= 0x7fffffffLL && tpt >= 2 && tpt <= 4) ? tpt : 0;
  const __amdgpu_buffer_rsrc_t orsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(out + u * out_su), 0, (int)min(oreach, (int64_t)0x7fffffff), 0x00020000);
  const int64_t my_off = my_row * out_si;
  auto emit_direct = [&](auto tptc) {
    constexpr int TPT = decltype(tptc)::value;
#pragma unroll
    for (int i = 0; i < ENC_TG; ++i)
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const int l = (tpend + i) * TPT + j;
        const bool ok = i < npend && l < l1 && my_ok;
        const uint32_t off = ok ? (uint32_t)(2 * ((int64_t)l * out_sl + my_off)) : 0x80000000u;
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)__builtin_amdgcn_ubfe(wd[i], (uint32_t)(K * j), (uint32_t)K),
                                              orsrc, off, 0, 0);
      }
  };
  // The stage loop is instantiated per path (general, and fast for each
  // tables-per-tile count), so that the compiler's wait analysis of one never
  // merges with another's.
  auto run_stages = [&](auto tptc) {
    constexpr int TPT = decltype(tptc)::value;  // 0: general path
    constexpr int NST = ENC_TG * (TPT > 0 ? TPT : 1);
    static_assert(NST < 64, "the vector-memory count of s_waitcnt has 6 bits");
    int buf = 0;
    for (int tg = t0; tg < t1; tg += ENC_TG) {
      const int tnext = tg + ENC_TG;
      const bool stores = TPT > 0 && npend;
      if constexpr (TPT > 0) {
        if (tnext < t1) MP_FETCH(buf ^ 1, tnext);
        asm volatile("" ::: "memory");
        if (npend) emit_direct(tptc);
        asm volatile("" ::: "memory");
      } else {
        if (npend) emit_stage();
        if (tnext < t1) MP_FETCH(buf ^ 1, tnext);
      }
      // every stage runs ENC_TG tiles (one straight block of matrix-core and
      // vector work for the scheduler; tiles past t1 read stale LDS and are
      // dropped).  The next tile's A operands are read from LDS while the
      // current tile's matrix-core ops run.
      // Software pipeline over the stage's tiles: tile tt's matrix-core ops
      // are issued before tile tt-1's sign bits are formed, so the vector
      // work of one tile runs while the matrix core works on the next.
      bf16x8 ap[2][KSTEPS];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) ap[0][s] = __builtin_bit_cast(bf16x8, wsh[buf][s * 64 + lane]);
      f32x16 acc[2][2];
#pragma unroll
      for (int tt = 0; tt <= ENC_TG; ++tt) {
        if (tt < ENC_TG) {
          if (tt + 1 < ENC_TG) {
#pragma unroll
            for (int s = 0; s < KSTEPS; ++s)
              ap[(tt + 1) & 1][s] = __builtin_bit_cast(bf16x8, wsh[buf][((tt + 1) * KSTEPS + s) * 64 + lane]);
          }
          // the next tile's operand reads stay ahead of this tile's
          // matrix-core ops (left to itself the scheduler moves each read
          // next to its use, and every pair of ops then waits for LDS)
          __builtin_amdgcn_sched_barrier(0);
          f32x16 a0 = {}, a1 = {};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) {
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[tt & 1][s], xb[0][s], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ap[tt & 1][s], xb[1][s], a1, 0, 0, 0);
          }
          acc[tt & 1][0] = a0;
          acc[tt & 1][1] = a1;
        }
        if (tt > 0) {
          const int tp = tt - 1;
          // lane l < 32 holds bits 0-15 of row l in m0 and bits 0-15 of row
          // 32 + l in m1; lane 32 + l holds bits 16-31 of the same rows.  One
          // cross-half swap leaves lane l with row l's halves and lane 32 + l
          // with row 32 + l's.
          uint32_t m0, m1;
          if constexpr (LIFT) {
            const int tl = min(tg + tp, t1 - 1);  // tiles past t1 are dropped
            const uint4 wl[2] = {wlift[tl * 4 + 2 * half], wlift[tl * 4 + 2 * half + 1]};
            m0 = sign_bits16_lift(acc[tp & 1][0], ebar[0], wl);
            m1 = sign_bits16_lift(acc[tp & 1][1], ebar[1], wl);
          } else {
            m0 = sign_bits16(acc[tp & 1][0]);
            m1 = sign_bits16(acc[tp & 1][1]);
          }
          const auto sw = __builtin_amdgcn_permlane32_swap(m0, m1, false, false);
          wd[tp] = sw[0] | (sw[1] << 16);
        }
      }
      tpend = tg;
      npend = min(ENC_TG, t1 - tg);
      if (stores) {
        // vmcnt(NST) lgkmcnt(0): this wave's projection copy (issued before
        // its NST code stores) has landed in LDS and its LDS reads are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt((NST & 15) | (7 << 4) | ((NST >> 4) << 14));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
      buf ^= 1;
    }
    if (npend) {
      if constexpr (TPT > 0)
        emit_direct(tptc);
      else
        emit_stage();
    }
  };
  if (ftpt == 3)
    run_stages(std::integral_constant<int, 3>{});
  else if (ftpt == 4)
    run_stages(std::integral_constant<int, 4>{});
  else if (ftpt == 2)
    run_stages(std::integral_constant<int, 2>{});
  else
    run_stages(std::integral_constant<int, 0>{});
#undef MP_FETCH
}

// ---------------------------------------------------------------------------
// Encoder for small jobs (at most 64 rows in all, e.g. the key appended per
// unit and the queries of a decode step).  A block takes SM_TABLES tables of
// one job; each of its 4 waves computes one of the (at most 3) tiles
// covering those tables.  A wave reads its tile's A operands straight from
// the packed projections (no LDS staging), holds all rows as the two 32-row
// B operands, and writes the 32 sign bits of every row for the tile to LDS;
// after one barrier each code is cut out of its row's bit string.  One memory
// round trip for the rows and projections, one for the codes.
constexpr int SM_TABLES = 4;                                   // tables per block
constexpr int SM_MAXT = 3;  // tiles a block touches: K <= 16 gives tpt >= 2, and 4 tables span <= 3 tiles
static_assert(SM_MAXT <= 4, "one tile per wave");

template <typename T, bool LIFT>
__global__ __launch_bounds__(256) void encode_small_kernel(EncJob j0, EncJob j1, int njobs, int blocks0,
                                                           const uint4 *__restrict__ wp, int K, int L,
                                                           const uint4 *__restrict__ wlift) {
  __shared__ uint32_t bits[64][SM_MAXT + 2];  // [row][tile - t0]
  touch_kernargs<7>();  // 400 bytes of arguments (two jobs of 184)
  const bool second = njobs > 1 && (int)blockIdx.x >= blocks0;
  const EncJob &jb = second ? j1 : j0;
  const int lb = second ? (int)blockIdx.x - blocks0 : (int)blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, half = lane >> 5;
  const int l0 = lb * SM_TABLES, l1 = min(L, l0 + SM_TABLES);
  const int tpt = enc_tpt(K);
  const int t0 = K > 0 ? l0 / tpt : 0, t1 = K > 0 ? (l1 + tpt - 1) / tpt : 0;
  const int R = (int)(jb.units * jb.rows);  // rows of the job, flattened (<= 64)
  const T *__restrict__ in = (const T *)jb.in;
  T *__restrict__ kcopy = (T *)jb.kcopy;
  const T *__restrict__ vin = (const T *)jb.vin;
  T *__restrict__ vcopy = (T *)jb.vcopy;
  // this wave's tile: its A operands are loaded first, so that their latency
  // overlaps the row loads
  const int t = t0 + wave;
  const bool has_tile = t < t1;
  uint4 a[KSTEPS];
  if (has_tile) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) a[s] = wp[((int64_t)t * KSTEPS + s) * 64 + lane];
  }

  // B operands: row r = 32 nt + lane % 32 (unit r / rows, row r % rows), dims
  // 16 s + 8 half + e.  All loads of a 32-row set go out before any is used;
  // rows past the job's last read its last row and are zeroed after.
  bf16x8 xb[2][KSTEPS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    if (nt == 1 && R <= 32) {  // no second row set
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[1][s][e] = (__bf16)0.0f;
      break;
    }
    const int r = 32 * nt + (lane & 31);
    const bool ok = r < R;
    const int rows = (int)jb.rows;  // rows of a small job fit an int
    const int rc = ok ? r : R - 1;
    const int64_t u = rc / rows, i = rc % rows;
    const T *rp = in + u * jb.in_su + i * jb.in_si + 8 * half;
    float v[KSTEPS][8];
    if (jb.mu) {
      const float *mp = jb.mu + u * jb.mu_su + i * jb.mu_si + 8 * half;
      float m[KSTEPS][8];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        load_row8<T>(rp + 16 * s, v[s]);
        load8<float>(mp + 16 * s, m[s]);
      }
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) v[s][e] = v[s][e] - m[s][e];  // fp32 subtraction
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) load_row8<T>(rp + 16 * s, v[s]);
    }
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[nt][s][e] = ok ? (__bf16)v[s][e] : (__bf16)0.0f;  // round to nearest even
  }
  // lifted rows: the extra coordinate of this lane's row of each set
  float ebar[2] = {0.0f, 0.0f};
  if constexpr (LIFT) {
    if (jb.rl) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int rr = min(32 * nt + (lane & 31), R - 1);
        const int64_t uu = rr / (int)jb.rows, ii = rr % (int)jb.rows;
        ebar[nt] = lift_coord(xb[nt], jb.rl[uu * jb.rl_su + ii * jb.rl_si]);
      }
    }
  }

  // appends: the job's blocks copy the raw key and value rows into the
  // caches, each its share of the 16-byte pieces (one per thread for up to
  // blocks0 * 256 pieces; both loads before both stores)
  if (kcopy && vcopy) {
    constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
    for (int c = lb * 256 + (int)threadIdx.x; c < R * CPR; c += blocks0 * 256) {
      const int r = c / CPR, pc = c % CPR;
      const int64_t u = r / (int)jb.rows, i = r % (int)jb.rows;
      const uint4 kx = *(const uint4 *)((const char *)(in + u * jb.in_su + i * jb.in_si) + 16 * pc);
      const uint4 vx = *(const uint4 *)((const char *)(vin + u * jb.in_su + i * jb.in_si) + 16 * pc);
      *(uint4 *)((char *)(kcopy + u * jb.kc_su + i * jb.kc_si) + 16 * pc) = kx;
      *(uint4 *)((char *)(vcopy + u * jb.kc_su + i * jb.kc_si) + 16 * pc) = vx;
    }
  }

  const bool two = R > 32;
  if (has_tile) {
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]), xb[0][s], acc0, 0, 0, 0);
    if (two) {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[s]), xb[1][s], acc1, 0, 0, 0);
    }
    // lane l ends with the tile's 32 bits of row l (as in the large encoder)
    uint32_t m0, m1;
    if constexpr (LIFT) {
      const uint4 wl[2] = {wlift[t * 4 + 2 * half], wlift[t * 4 + 2 * half + 1]};
      m0 = sign_bits16_lift(acc0, ebar[0], wl);
      m1 = two ? sign_bits16_lift(acc1, ebar[1], wl) : 0u;
    } else {
      m0 = sign_bits16(acc0);
      m1 = two ? sign_bits16(acc1) : 0u;
    }
    const auto sw = __builtin_amdgcn_permlane32_swap(m0, m1, false, false);
    const uint32_t word = sw[0] | (sw[1] << 16);
    bits[lane][t - t0] = word;
  }
  __syncthreads();

  // codes: table l of row r is the bit field [K (l % tpt), + K) of the row's
  // word of tile l / tpt (all zero when K = 0)
  const int ntab = l1 - l0;
  for (int idx = threadIdx.x; idx < R * ntab; idx += 256) {
    const int r = idx / ntab, l = l0 + idx % ntab;
    const uint32_t c = K > 0 ? __builtin_amdgcn_ubfe(bits[r][l / tpt - t0], (uint32_t)(K * (l % tpt)), (uint32_t)K) : 0u;
    const int64_t u = r / (int)jb.rows, i = r % (int)jb.rows;
    jb.out[u * jb.out_su + (int64_t)l * jb.out_sl + i * jb.out_si] = (uint16_t)c;
  }
}

// Grid shape of one job.  Few rows: the tables are split over blocks so that
// the projection pass runs on many compute units instead of one.
static void plan_job(EncJob &j, int K, int L, int64_t first_block) {
  j.rblocks = (j.rows + ENC_ROWS - 1) / ENC_ROWS;
  const int64_t blocks = j.rblocks * j.units;
  int tsplit = 1;
  if (blocks < 512) tsplit = (int)std::min<int64_t>((512 + blocks - 1) / blocks, (int64_t)L);
  const int tpt = std::max(enc_tpt(K), 1);  // a block's tables start on a tile
  j.tpb = (L + tsplit - 1) / tsplit;
  j.tpb = (j.tpb + tpt - 1) / tpt * tpt;
  j.tsplit = (L + j.tpb - 1) / j.tpb;
  j.first_block = first_block;
}

static int64_t job_blocks(const EncJob &j) { return j.rblocks * j.units * j.tsplit; }

hipError_t launch_encode_jobs(int dtype, EncJob *jobs, int njobs, const void *Wp, int K, int L, hipStream_t s,
                              const uint16_t *wlift) {
  int64_t total = 0;
  EncJob j[2];
  int nj = 0;
  for (int i = 0; i < njobs; ++i) {
    if (jobs[i].units == 0 || jobs[i].rows == 0) continue;
    j[nj] = jobs[i];
    plan_job(j[nj], K, L, total);
    total += job_blocks(j[nj]);
    ++nj;
  }
  if (nj == 0) return hipSuccess;
  if (nj == 1) j[1] = j[0];
  bool small = true;
  for (int i = 0; i < nj; ++i) small = small && j[i].units * j[i].rows <= 64;
  const uint4 *wl = (const uint4 *)wlift;
  const bool lift = wlift != nullptr && K > 0;
#define MP_ENC(KERNEL, G, B, ...)                                                           \
  do {                                                                                      \
    if (dtype == 0 && lift)                                                                 \
      KERNEL<__bf16, true><<<G, B, 0, s>>>(__VA_ARGS__, wl);                                \
    else if (dtype == 0)                                                                    \
      KERNEL<__bf16, false><<<G, B, 0, s>>>(__VA_ARGS__, wl);                               \
    else if (lift)                                                                          \
      KERNEL<float, true><<<G, B, 0, s>>>(__VA_ARGS__, wl);                                 \
    else                                                                                    \
      KERNEL<float, false><<<G, B, 0, s>>>(__VA_ARGS__, wl);                                \
  } while (0)
  if (small) {
    const int bpj = (L + SM_TABLES - 1) / SM_TABLES;
    const dim3 g((unsigned)(bpj * nj));
    MP_ENC(encode_small_kernel, g, 256, j[0], j[1], nj, bpj, (const uint4 *)Wp, K, L);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)total);
  MP_ENC(encode_kernel, grid, 64 * ENC_NW, j[0], j[1], nj, (const uint4 *)Wp, K, L);
#undef MP_ENC
  return hipGetLastError();
}

hipError_t launch_encode(int dtype, const void *in, int64_t in_su, int64_t in_si, const float *mu, int64_t mu_su,
                         int64_t mu_si, int64_t units, int64_t rows, const void *Wp, int K, int L, uint16_t *out,
                         int64_t out_su, int64_t out_si, int64_t out_sl, void *kcopy, int64_t kc_su, int64_t kc_si,
                         const void *vin, void *vcopy, hipStream_t s) {
  EncJob j = make_job(in, in_su, in_si, mu, mu_su, mu_si, units, rows, out, out_su, out_si, out_sl, kcopy, kc_su,
                      kc_si, vin, vcopy);
  return launch_encode_jobs(dtype, &j, 1, Wp, K, L, s);
}

}  // namespace mp
