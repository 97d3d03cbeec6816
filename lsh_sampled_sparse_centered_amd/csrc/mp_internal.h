// Internal declarations shared by the HIP sources of libmagicpig.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;          // supported head dimension
constexpr int KSTEPS = D / 16;  // k-steps of one 32x32x16 bf16 matrix-core op over d

// ---------------------------------------------------------------- encoder
// Packed projections: [ntiles][KSTEPS][64 lanes][8 bf16], one 32-column tile
// = 8 KB.  A tile holds whole tables: tpt = floor(32 / K) tables per tile,
// table t*tpt + j in bits K*j .. K*j + K-1 of the tile's 32-bit word (the
// bits past tpt*K are zero columns).  Within a tile, matrix row i (the
// A-operand row that lane i % 32 supplies) carries word bit enc_row_col(i);
// the order is chosen so that accumulator register r of lane half a holds
// bit 16*a + r, i.e. each lane's 16 sign bits come out in bit order.
constexpr int ENC_NW = 4;       // waves per encoder block (64 rows each)
constexpr int ENC_ROWS = 64 * ENC_NW;  // rows (keys or queries) per encoder block
#ifndef MP_ENC_OCC
#define MP_ENC_OCC 2  // encoder waves per SIMD the kernel is compiled for
#endif
#ifndef MP_ENC_TG
#define MP_ENC_TG 2
#endif
constexpr int ENC_TG = MP_ENC_TG;  // tiles staged in LDS per stage (8 KB each, double buffered)
constexpr int ENC_CST = (ENC_TG - 1) * 8 + 8;  // LDS code slots per wave and stage (8 per tile)
__host__ __device__ inline int enc_tpt(int K) { return K > 0 ? 32 / K : 0; }
__host__ __device__ inline int enc_ntiles(int K, int L) { return K > 0 ? (L + enc_tpt(K) - 1) / enc_tpt(K) : 0; }
__host__ __device__ inline int enc_row_col(int i) { return 16 * ((i >> 2) & 1) + (i & 3) + 4 * (i >> 3); }

// ---------------------------------------------------------------- decode
constexpr int SCAN_TILE = 512;  // keys per scan tile: 64 lanes x 8 keys (16 B of codes per table)
constexpr int PSTRIDE = 132;    // floats per partial record: m, l, count, pad, o[128]
constexpr int MAX_G = 8;        // query heads per KV head handled by one pass
constexpr int MAX_L = 512;

// Sampling-probability constants for one (L, T), filled on the host: series
// coefficients a[i] = C(L, 2+i) / C(L, 2) and lnc2 = ln C(L, 2) for the
// pages' threshold T = 2, and lnct = ln C(L, T) for other thresholds.
constexpr int LNP_TERMS = 12;
struct LnPCoef {
  float a[LNP_TERMS];
  float lnc2;
  float lnct;
  int T;  // collision threshold: a key is sampled in at least T of L tables
  float Kf, Lf, Lm1, Lm2, Tf, LmT;  // K, L, L - 1, L - 2, T, L - T as floats (no conversions in the kernel)
};
LnPCoef lnp_coef(int K, int L, int T);

struct DecodeGeom {
  int64_t U;          // units = B * Hkv
  int64_t chunk;      // keys per block = chunk_tiles * SCAN_TILE
  int64_t nchunks;    // blocks per unit for this n
  int64_t nchunks_max;  // for n = cap (workspace sizing)
};

// Workspace layout of the decode: [qcodes B*Hq*L u16, 256-aligned]
// [partials U * nchunks_max * G * PSTRIDE f32] [entries U * nchunks_max * chunk u32]
// [entry counts U * nchunks_max i32] [sampled-key bitmaps U * G * nchunks_max * 16 u32].
struct DecodeWs {
  uint16_t *qcodes;
  float *part;
  uint32_t *ent;
  int32_t *ent_cnt;
  uint32_t *bits;  // per (unit, head) one bit per key: sampled (bucket lookup)
  size_t bytes;
};

DecodeGeom decode_geom(int B, int Hkv, int Hq, int64_t n, int64_t cap);
// Tiles with bucket-lookup bitmaps taken SPAN_TILES per sampling block (one
// or two query heads per unit, bf16 caches) when one tile per block would
// make a grid of at least SPAN_MIN_BLOCKS blocks, four times what the chip
// keeps resident (256 compute units x 7 blocks): one prologue per block and
// fuller attention rounds.  The block's record goes to its first tile's
// slot, empty records (m = -inf, l = 0) to the others.
constexpr int SPAN_TILES = 4;
constexpr int64_t SPAN_MIN_BLOCKS = 4 * 256 * 7;
// Bitmap tiles per sampling block for a launch (dtype 0: bf16 caches; nlt:
// tiles with bitmaps).
inline int sample_span(int dtype, int G, int64_t nlt, const DecodeGeom &g) {
  return (dtype == 0 && G <= 2 && nlt >= 2 && g.U * g.nchunks >= SPAN_MIN_BLOCKS) ? SPAN_TILES : 1;
}
DecodeWs decode_ws_layout(void *base, int B, int Hq, int Hkv, int64_t cap, int L);

// Launchers (defined in the .hip files); they return hipError_t of the launch.
hipError_t launch_proj_pack(const float *W, int K, int L, void *Wp, hipStream_t s);
hipError_t launch_kmean(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, double *partial,
                        int nparts, float *kmean, hipStream_t s);
int kmean_parts(int64_t n);
// One encoder row set: row i of unit u is read at in + u*in_su + i*in_si
// (elements), centred by mu + u*mu_su + i*mu_si when mu is set, and its code
// of table l written to out + u*out_su + i*out_si + l*out_sl; when kcopy is
// set the raw row (and vin's row) are also copied to kcopy/vcopy + u*kc_su +
// i*kc_si.  The launcher fills the grid fields.
// A kernel's explicit arguments span LINES 64-byte lines, which the compiler
// loads where each is first used -- a chain of dependent scalar loads, each
// a memory round trip when it misses.  One scalar load per line at entry
// brings them in together (reads only; every line touched starts inside the
// explicit arguments).
template <int LINES>
__device__ inline void touch_kernargs() {
  typedef const __attribute__((address_space(4))) uint32_t karg_t;
  karg_t *kp = (karg_t *)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < LINES; ++i) x ^= kp[16 * i];
  asm volatile("" ::"s"(x));
}

struct EncJob {
  const void *in;
  int64_t in_su, in_si;
  const float *mu;
  int64_t mu_su, mu_si;
  int64_t units, rows;
  uint16_t *out;
  int64_t out_su, out_si, out_sl;
  void *kcopy;
  int64_t kc_su, kc_si;
  const void *vin;
  void *vcopy;
  const float *rl;  // lifted rows (Equation 8): row i of unit u has radius rl[u*rl_su + i*rl_si]; NULL: not lifted
  int64_t rl_su, rl_si;
  int64_t rblocks, first_block;
  int tsplit, tpb;
};

inline EncJob make_job(const void *in, int64_t in_su, int64_t in_si, const float *mu, int64_t mu_su, int64_t mu_si,
                       int64_t units, int64_t rows, uint16_t *out, int64_t out_su, int64_t out_si, int64_t out_sl,
                       void *kcopy, int64_t kc_su, int64_t kc_si, const void *vin, void *vcopy) {
  EncJob j{};
  j.in = in;
  j.in_su = in_su;
  j.in_si = in_si;
  j.mu = mu;
  j.mu_su = mu_su;
  j.mu_si = mu_si;
  j.units = units;
  j.rows = rows;
  j.out = out;
  j.out_su = out_su;
  j.out_si = out_si;
  j.out_sl = out_sl;
  j.kcopy = kcopy;
  j.kc_su = kc_su;
  j.kc_si = kc_si;
  j.vin = vin;
  j.vcopy = vcopy;
  return j;
}

// Encodes up to two row sets in one launch.  wlift (lifted rows only): the
// projections' extra row, [ntiles][32] bf16 in tile-word bit order.
hipError_t launch_encode_jobs(int dtype, EncJob *jobs, int njobs, const void *Wp, int K, int L, hipStream_t s,
                              const uint16_t *wlift = nullptr);
// Lift radius per unit (Equation 8): rlift[u] = fp32(sqrt(max_i |bf16(K[u][i] - kmean[u])|^2)), fp64 sums.
hipError_t launch_lift_radius(const void *Kc, int kv_dtype, int64_t U, int64_t n, int64_t cap, const float *kmean,
                              double *partial, int nparts, float *rlift, hipStream_t s);
hipError_t launch_proj_pack_lift(const float *W, int K, int L, uint16_t *wlift, hipStream_t s);
hipError_t launch_encode(int dtype, const void *in, int64_t in_su, int64_t in_si, const float *mu, int64_t mu_su,
                         int64_t mu_si, int64_t units, int64_t rows, const void *Wp, int K, int L, uint16_t *out,
                         int64_t out_su, int64_t out_si, int64_t out_sl, void *kcopy, int64_t kc_su, int64_t kc_si,
                         const void *vin, void *vcopy, hipStream_t s);
// When ev_start / ev_stop are set they are attached to the kernel's own
// dispatch, so they time exactly this launch (no queue gap before it).
// Tiles below n_lists take their sampled keys from the workspace's bitmaps
// (written by launch_bucket_lookup) instead of scanning.
// rlift (nullable, [U]): the keys were hashed lifted (Equation 8) with these
// radii, and the sampling angle is taken against the lifted key.
hipError_t launch_sample(int dtype, const void *q, const void *Kc, const void *Vc, const uint16_t *codes,
                         const float *kmean, const uint16_t *qcodes, int B, int Hq, int Hkv, int64_t n, int64_t cap,
                         int K, int L, int T, int64_t nsh, int64_t nst, const DecodeGeom &geo, const DecodeWs &ws,
                         bool want_idx, hipStream_t s, hipEvent_t ev_start = nullptr,
                         hipEvent_t ev_stop = nullptr, const uint32_t *planes = nullptr, int64_t n_planes = 0,
                         int64_t n_lists = 0, const float *rlift = nullptr);
// Bit-plane index of the code store: tiles [t0, t0 + nt) of every unit,
// planes [U][ptiles][K][L][16] u32 (word j of row (b, l) of tile t = bit b of
// table l's codes for keys 512 t + 32 j .. + 31).
hipError_t launch_plane_build(const uint16_t *codes, int64_t U, int64_t cap, int K, int L, int64_t t0, int64_t nt,
                              uint32_t *planes, hipStream_t s);
// With (nlt, span) from the sampling launch, the merge reads only the
// records that launch filled (one per block); with the defaults it reads
// every tile's (the empty ones weigh nothing).
hipError_t launch_merge(int B, int Hq, int Hkv, int64_t n, int L, const DecodeGeom &geo, const DecodeWs &ws,
                        float *out, float *lse, int32_t *idx, int64_t cap, int32_t *count, hipStream_t s,
                        int64_t nlt = 0, int span = 1);

// ---------------------------------------------------------------- bucketed tables
// Per (unit, table, chunk of BK_R keys) a table of 2^K buckets: the chunk's
// keys ordered by their code (CSR).  off [U][L][2^K][bchunks] uint32: word
// (u, l, c, r) = start | count << 16 of bucket c in chunk r (its entries
// are keys[u][l][r * BK_R + start ..]; the words of one bucket over all
// chunks are adjacent, so a lookup of a (unit, head, table) touches one
// line of offsets); keys [U][L][cap] uint16 (the key's offset from its
// chunk's first key).
constexpr int BK_R = 8192;  // keys per bucket chunk (16 scan tiles); starts and counts fit 16 bits
constexpr int MAX_BK_K = 12;  // bits per table the bucketed tables support (2^K buckets per chunk)
struct BucketLayout {
  uint32_t *off;
  uint16_t *keys;
  int64_t bchunks;  // chunks per unit for the capacity
  int nbins;        // 2^K
  size_t bytes;
};
BucketLayout bucket_layout(void *base, int64_t U, int64_t cap, int K, int L);
// (Re)builds the chunks [n0 / BK_R, ceil(n1 / BK_R)) from the codes of keys [.., n1).
hipError_t launch_bucket_build(const uint16_t *codes, int64_t U, int64_t cap, int K, int L, int64_t n0, int64_t n1,
                               const BucketLayout &bl, hipStream_t s);
// Sampled-key bitmaps (threshold 2) of the tiles below nb (a multiple of
// SCAN_TILE), from the query codes' buckets, into the workspace's bitmaps.
// ev_start, when set, is attached to the lookup's own dispatch (its start).
hipError_t launch_bucket_lookup(const uint16_t *qcodes, const BucketLayout &bl, int B, int Hq, int Hkv, int64_t n,
                                int64_t nb, int64_t cap, int K, int L, int64_t nsh, int64_t nst, const DecodeGeom &geo,
                                const DecodeWs &ws, hipStream_t s, hipEvent_t ev_start = nullptr);

}  // namespace mp
