// Fast paths for n = 4 bfloat16 streams on gfx950.
//
// mhc_split_kernel<POST> streams the state in 256-channel super-chunks of
// 32-token tiles:
//   POST: X_next = h_res X + h_post^T F_out  (mHC notes Eq. 3, F_post,res of 4.3.1)
//   always: the skinny projection of the state it streams (the X_next it just
//         produced when POST, else X) with MFMA, and the sum of squares.
// proj_wide_kernel is the projection alone on 64-token items (up to 24
// columns): each phi fragment read from L2 serves twice the tokens.
// coeffs_finish_kernel turns the projections into the coefficients (Eq. 15-19):
// RMS factor, gates, sigmoid, 2*sigmoid and Sinkhorn-Knopp.
// The projection uses v_mfma_f32_16x16x32_bf16 with 16 tokens as the M rows. phi (float32) is split as phi = hi + lo with hi = bf16(phi) and
// lo = bf16(phi - hi), so X (exact in bf16) times hi plus X times lo carries
// about 16 significant bits of phi into an fp32 accumulator. phi is packed once
// per call into the B-operand order [row/8][48][8] (hi columns 0..23, lo
// columns 24..47), so each lane's 8 k-values of one column are 16 contiguous
// bytes.
#include <type_traits>

#include "hc_device.h"
#include "hc_fast.h"
#include "hc_launch.h"

namespace hc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int NS4 = 4;              // streams
constexpr int NCOL = 24;            // n*n + 2n
constexpr int TOK = 16;             // tokens per tile (MFMA M)

// ------------------------------------------------------------- phi packing

// phi_a [K, na] | phi_b [K, nb] (nb may be 0) -> the packed B-operand form: per
// group of 8 rows, 2 ncolp columns of 8 bf16, columns 0..ncolp-1 hi = bf16(phi)
// and ncolp..2 ncolp-1 lo = bf16(phi - hi); columns past na + nb are zero. One
// workgroup per 64 rows (K is a multiple of 64 on the fast paths): the rows are
// read into LDS, then thread (row group g, column c) writes the two chunks.
// With rows_out (the mHC backward, nc <= 32), thread (row t >> 2, column group
// t & 3) also writes the row form: per row 128 bytes, bf16 hi of columns 0..31
// then bf16 lo (the B operand of dP phi^T: one row, 8 consecutive columns).
// 8 consecutive rows of one column -> hi = bf16(p) and lo = bf16(p - hi) (p - hi is
// exact in float32), 8 bf16 each.
__device__ __forceinline__ void pack8_hilo(const float p[8], uint4& hi_out, uint4& lo_out) {
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const uint32_t h0 = f2bf(p[e]), h1 = f2bf(p[e + 1]);
    hi[e / 2] = h0 | (h1 << 16);
    lo[e / 2] = f2bf(p[e] - bf2f(h0)) | (f2bf(p[e + 1] - bf2f(h1)) << 16);
  }
  hi_out = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  lo_out = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

__global__ __launch_bounds__(256) void pack_phi_kernel(const float* __restrict__ phi_a, int na,
                                                       const float* __restrict__ phi_b, int nb, int ncolp,
                                                       uint16_t* __restrict__ packed, uint4* __restrict__ rows_out) {
  __shared__ float rows[64 * 32];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int nc = na + nb;
  for (int i = threadIdx.x; i < 64 * nc; i += 256) {
    const int r = i / nc, c = i - r * nc;
    rows[r * 32 + c] = c < na ? phi_a[(r0 + r) * na + c] : phi_b[(r0 + r) * nb + (c - na)];
  }
  __syncthreads();
  if (rows_out) {
    const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float a = q * 8 + e < nc ? rows[r * 32 + q * 8 + e] : 0.f;
      const float b = q * 8 + e + 1 < nc ? rows[r * 32 + q * 8 + e + 1] : 0.f;
      const uint32_t h0 = f2bf(a), h1 = f2bf(b);
      hi[e / 2] = h0 | (h1 << 16);
      lo[e / 2] = f2bf(a - bf2f(h0)) | (f2bf(b - bf2f(h1)) << 16);
    }
    rows_out[(r0 + r) * 8 + q] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    rows_out[(r0 + r) * 8 + 4 + q] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  if ((int)threadIdx.x >= 8 * ncolp) return;
  const int g = threadIdx.x / ncolp, c = threadIdx.x - g * ncolp;
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = c < nc ? rows[(g * 8 + e) * 32 + c] : 0.f;
  uint4* out = reinterpret_cast<uint4*>(packed) + (r0 / 8 + g) * (2 * ncolp);
  pack8_hilo(p, out[c], out[ncolp + c]);
}

// The same packed form for the columns of up to 5 row-major sources [K, nc_j]
// placed side by side (at most 80 columns): the xHC-Flash block entry packs the
// router and the L pre maps into one operand.
struct PackSrcs {
  const float* p[5];
  int nc[5];
  int ns;
};
constexpr int PACK_MAXC = 80;
__global__ __launch_bounds__(256) void pack_phi_multi_kernel(PackSrcs S, int ncolp, uint16_t* __restrict__ packed) {
  __shared__ float rows[64 * PACK_MAXC];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  // 4 threads per row: source j's columns of row r are read at c = (tid & 3) + 4 i,
  // so the threads of a workgroup read each source's 64 rows as one contiguous block
  const int r = threadIdx.x >> 2, c4 = threadIdx.x & 3;
  int nc = 0;
  for (int j = 0; j < S.ns; ++j) {
    const float* src = S.p[j] + (r0 + r) * S.nc[j];
    for (int c = c4; c < S.nc[j]; c += 4) rows[r * PACK_MAXC + nc + c] = src[c];
    nc += S.nc[j];
  }
  __syncthreads();
  for (int w = threadIdx.x; w < 8 * ncolp; w += 256) {
    const int g = w / ncolp, c = w - g * ncolp;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) p[e] = c < nc ? rows[(g * 8 + e) * PACK_MAXC + c] : 0.f;
    uint4* out = reinterpret_cast<uint4*>(packed) + (r0 / 8 + g) * (2 * ncolp);
    pack8_hilo(p, out[c], out[ncolp + c]);
  }
}

// ---------------------------------------------------------- stream kernel

struct Gate {
  float a_pre, a_post, a_res;
};

__device__ __forceinline__ uint32_t bf16_lo(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t bf16_hi(uint32_t w) { return w & 0xffff0000u; }

__device__ __forceinline__ void unpack8(const uint4& q, float v[8]) {
  v[0] = __uint_as_float(bf16_lo(q.x)); v[1] = __uint_as_float(bf16_hi(q.x));
  v[2] = __uint_as_float(bf16_lo(q.y)); v[3] = __uint_as_float(bf16_hi(q.y));
  v[4] = __uint_as_float(bf16_lo(q.z)); v[5] = __uint_as_float(bf16_hi(q.z));
  v[6] = __uint_as_float(bf16_lo(q.w)); v[7] = __uint_as_float(bf16_hi(q.w));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& q) {
  return __builtin_bit_cast(bf16x8_t, q);
}

// Work split of one workgroup (32 tokens = two 16-row MFMA blocks, 512 threads
// = 8 waves) per 256-channel super-chunk of all 4 streams of a tile:
//  * streaming phase: thread (token tid>>5 and tid>>5 + 16, 8 channels at
//    (tid&31)*8) loads its 16-byte pieces of the 4 streams (and of F_out), so 32
//    consecutive lanes read 512 contiguous bytes of one stream row; with POST it
//    computes and stores X_next; the bf16 tile it projects (X_next or X) goes to
//    LDS;
//  * MFMA phase: wave w takes the 32-channel group w of the super-chunk for all
//    4 streams, loads that group's B fragments once and applies them to both
//    token blocks, whose A fragments (16 tokens x 32 k) it reads from LDS.
// LDS is double-buffered (one barrier per super-chunk) and the next
// super-chunk's loads are in flight during the current one.
constexpr int SC = 256;                 // channels per super-chunk
constexpr int SWAVE = 8;                // waves per workgroup
constexpr int STHR = SWAVE * 64;
constexpr int TILE = 2 * TOK;           // tokens per workgroup
constexpr int LROW = SC * 2 + 16;       // bytes per (stream, token) row in LDS, padded
constexpr int LBUF = NS4 * TILE * LROW; // bytes per LDS buffer

// Loads of the streamed state (read once per pass): nontemporal, so they stream
// through L2 without displacing the packed phi that every item re-reads.
__device__ __forceinline__ uint4 ld_stream(const uint16_t* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// v if keep, else zeros: per-component selects (a select between two uint4
// objects can become a select of their addresses, which puts them in scratch).
__device__ __forceinline__ uint4 keep_or_zero(bool keep, const uint4& v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// Work items: a tile of 32 tokens times a group of 4 streams times a slice of
// SPI super-chunks (SPI * 256 channels). Items are numbered tile-major and a
// persistent grid of one workgroup per CU takes items blockIdx.x, blockIdx.x +
// grid, ..., so at any moment the running workgroups cover a few adjacent tiles
// entirely: a compact window of HBM. (Giving each workgroup a whole tile
// instead puts 256 strips of 512 bytes per 8 KB stream row in flight across
// the whole state, which streams about 10% slower.) Each item leaves its
// partial projection, [32 tokens][NB*8 columns | sum of squares] in float, in a
// workspace; the finish kernels add a tile's items in a fixed order.
//
// Which 4 streams an item reads (MODE):
//   ROWS_CONTIG: the token row is the 4 streams (mHC state [T, 4, C]);
//   ROWS_GROUPS: streams 4g..4g+3 of a wider row (xHC full state [T, N, C],
//                N = 4 NG), with phi rows of those streams;
//   ROWS_GATHER: the streams idx[t, 0..3] of a token row (xHC active set), with
//                phi rows of slots 0..3.
//
// proj_wide_kernel (64-token items) takes ROWS_GATHER (with up to 32 columns) and two more:
//   ROWS_DENSE: all 16 streams of the xHC full state, item = 64 tokens x 256
//                channels of every stream group (the groups are the inner
//                steps); it also forms the dense read F_in = sum_i h_pre_i x_i
//                of the rows it streams, and leaves the rows idx[t, 0..3] out
//                of the projection;
//   ROWS_PAIRS:  one stream row per item token: token m of pair tile p is the
//                row (ptok[64 p + m], bucket stream of the tile), its 4 quarter
//                rows taking the place of the 4 streams (phi rows of that
//                stream); ptok < 0 marks padding.
constexpr int SPI = 4;                   // super-chunks per item
constexpr int NCOEF = TILE * 20;         // h_res (16) | h_post (4) per token of a tile
enum : int { ROWS_CONTIG = 0, ROWS_GROUPS = 1, ROWS_GATHER = 2, ROWS_DENSE = 3, ROWS_PAIRS = 4 };

template <int NB, int TT = TILE, int EX = 0>  // TT: tokens per item; EX: extra columns after ss
struct PartGeom {
  static constexpr int NCP = NB * 16;         // packed hi | lo columns
  static constexpr int NCOLP = NB * 8;        // logical columns (padded)
  static constexpr int PROW = NCOLP + 1 + EX; // floats per token of a partial: columns | ss | EX extra
  static constexpr int PART = TT * PROW;
  static constexpr int NPEND = (PART + STHR - 1) / STHR;
};

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N - 1>{})
template <int N, typename Fn, int I = 0>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, Fn, I + 1>(static_cast<Fn&&>(f));
  }
}

// Buffer resource over [base, base + bytes): stores whose offset falls outside are
// dropped by the hardware, so a guarded store needs no branch (a store behind a
// branch makes the compiler's wait counts conservative at the merge).
constexpr unsigned BUF_DW3 = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;  // any offset >= the range is dropped

struct SplitArgs {
  const uint16_t* X;
  int64_t T, C;
  int64_t rowstride;  // elements per token row of X
  int NG, S, nitem;   // stream groups, slices per group, items
  const int32_t* idx; // ROWS_GATHER: [T, kidx] stream indices (slots 0..3 used)
  int kidx, nstreams; // idx row length; streams per row (indices are clamped into range)
  const float* h_res_in;   // POST: [T, 16]
  const float* h_post_in;  // POST: [T, 4]
  const uint16_t* F;       // POST: [T, C]
  uint16_t* Y;             // POST: [T, 4, C]
  const uint16_t* phi_p;   // packed phi, NB * 16 columns
  float* part;             // [nitem][tokens per item][PROW]
  const uint16_t* dF;      // proj_wide_kernel with DH: dF_in [T, C]
  const float* hd;         // ROWS_DENSE: h_pre [T, 16] of the dense read
  uint16_t* Fd;            // ROWS_DENSE: the dense read's output F_in [T, C]
  const int32_t* ptok;     // ROWS_PAIRS: token of each pair [ntile * 64] (< 0: padding)
  const int32_t* tile_off; // ROWS_PAIRS: [nstreams + 1] first pair tile of each stream's bucket
  int64_t sq;              // ROWS_PAIRS: elements between consecutive streams of a token row
};

template <bool POST, int NB, int MODE>
__global__ __launch_bounds__(STHR) void mhc_split_kernel(SplitArgs A) {
  static_assert(!POST || MODE == ROWS_CONTIG, "the post/res write is for the mHC state");
  static_assert(MODE <= ROWS_GATHER, "dense and pair rows use proj_wide_kernel");
  static_assert(SPI >= 3, "the next item's stream table is written after the second super-chunk");
  using PG = PartGeom<NB>;
  constexpr int NCP = PG::NCP;
  const uint16_t* X = A.X;
  const int64_t T = A.T, C = A.C;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * LBUF];
  // coefficients of the tile being streamed and of the next item's tile
  __shared__ float coef[POST ? 2 * NCOEF : 1];
  // stream indices of the tile being streamed and of the next item's tile
  __shared__ __attribute__((aligned(16))) int gtab[MODE == ROWS_GATHER ? 2 * TILE * 4 : 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // streaming-phase role: tokens st_tok and st_tok + 16 of the tile, 8 channels
  const int st_tok = tid >> 5;
  const int st_c8 = (tid & 31) * 8;
  // MFMA-phase role
  const int tau = lane & 15;
  const int q = lane >> 4;
  const int G = (int)gridDim.x;
  const int nk = (A.nitem - (int)blockIdx.x + G - 1) / G;  // items of this workgroup (>= 1)
  const int per_tile = A.NG * A.S;

  floatx4_t acc[2][NB], gram[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    gram[tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const __amdgpu_buffer_rsrc_t pres =
      __builtin_amdgcn_make_buffer_rsrc(A.part, 0, (uint32_t)((int64_t)A.nitem * PG::PART * 4), BUF_DW3);

  // coefficient cidx (< NCOEF) of a tile; rows past T are clamped (never used)
  auto coef_val = [&](int tile, int cidx) __attribute__((always_inline)) {
    const int m = cidx / 20, e = cidx - m * 20;
    int64_t tt = (int64_t)tile * TILE + m;
    tt = tt < T ? tt : T - 1;
    const float* src = e < 16 ? A.h_res_in + tt * 16 + e : A.h_post_in + tt * 4 + (e - 16);
    return *src;
  };
  const int cidx1 = tid + STHR < NCOEF ? tid + STHR : NCOEF - 1;
  // stream index (slot tid & 3 of token tid >> 2, tid < 128) of a tile, clamped into range
  auto gidx_val = [&](int tile) __attribute__((always_inline)) {
    const int tt0 = tid < TILE * 4 ? tid : TILE * 4 - 1;
    int64_t tt = (int64_t)tile * TILE + (tt0 >> 2);
    tt = tt < T ? tt : T - 1;
    const int v = A.idx[tt * A.kidx + (tt0 & 3)];
    return v < 0 ? 0 : (v >= A.nstreams ? A.nstreams - 1 : v);
  };

  // Item geometry: tile, stream group, first super-chunk.
  struct Item {
    int tile, g;
    int64_t s0;
  };
  auto item_of = [&](int item) __attribute__((always_inline)) {
    const int tile = item / per_tile;
    const int r = item - tile * per_tile;
    const int g = r / A.S;
    return Item{tile, g, (int64_t)(r - g * A.S) * SPI};
  };

  // Loads are unconditional: rows past T and channels past C are clamped to a
  // valid address and their values replaced by zeros (or their stores dropped),
  // so no load sits behind a branch and consecutive loads stay in flight together.
  auto load_half = [&](const Item& it, int64_t s, const int* gt, auto P, uint4 (&xv)[NS4], uint4& fv)
                       __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int m = st_tok + 16 * p;
    int64_t t = (int64_t)it.tile * TILE + m;
    t = t < T ? t : T - 1;
    const int64_t c = s * SC + st_c8;
    const int64_t cc = c < C ? c : C - 8;
    const uint16_t* xr = X + t * A.rowstride + cc;
    if (MODE == ROWS_GATHER) {
      // Ordinary (cache-allocating) loads for the gathered rows: the mix pass that
      // follows reads the same rows again and finds part of them in the
      // last-level cache (measured when K = 4 routes took this kernel: 207.8
      // against 235.5 us per call at N = 16, C = 4096, T = 8192 with
      // nontemporal loads here).
      const int4 sv = *reinterpret_cast<const int4*>(gt + m * 4);
      xv[0] = *reinterpret_cast<const uint4*>(xr + (int64_t)sv.x * C);
      xv[1] = *reinterpret_cast<const uint4*>(xr + (int64_t)sv.y * C);
      xv[2] = *reinterpret_cast<const uint4*>(xr + (int64_t)sv.z * C);
      xv[3] = *reinterpret_cast<const uint4*>(xr + (int64_t)sv.w * C);
    } else {
      const uint16_t* xg = xr + (int64_t)(MODE == ROWS_GROUPS ? 4 * it.g : 0) * C;
#pragma unroll
      for (int i = 0; i < NS4; ++i) xv[i] = ld_stream(xg + i * C);
    }
    if (POST) fv = ld_stream(A.F + t * C + cc);
  };

  // Streaming work of one token half: X_next (POST) and the bf16 tile it
  // projects, into LDS.
  auto stream_half = [&](const Item& it, int64_t s, auto P, const uint4 (&xc)[NS4], const uint4& fc,
                         unsigned char* buf, const float* cf, __amdgpu_buffer_rsrc_t yres)
                         __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int m = st_tok + 16 * p;
    const int64_t c = s * SC + st_c8;
    const bool ok = ((int64_t)it.tile * TILE + m < T) && c < C;
    uint4 a_frag[NS4];
    if (POST) {
      const float* cm = cf + m * 20;
      float fv[8];
      unpack8(fc, fv);
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        float y[8];
        const float wp = cm[16 + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = wp * fv[e];
#pragma unroll
        for (int j = 0; j < NS4; ++j) {
          float xv[8];
          unpack8(xc[j], xv);
          const float w = cm[i * 4 + j];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] += w * xv[e];
        }
        uint4 o;
        o.x = pack_bf2_hw(y[0], y[1]);
        o.y = pack_bf2_hw(y[2], y[3]);
        o.z = pack_bf2_hw(y[4], y[5]);
        o.w = pack_bf2_hw(y[6], y[7]);
        a_frag[i] = o;  // positions past T or C are zeroed in the MFMA phase
        const uint32_t yoff = ok ? (uint32_t)((((int64_t)m * NS4 + i) * C + c) * 2) : OOB;
        // A cached store, not a nontemporal one: the pre-read that follows reads
        // these rows back newest first and finds many of them in the last-level
        // cache (on the 4 x 4096 state, about 9% off the whole call).
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{o.x, o.y, o.z, o.w}, yres, yoff, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NS4; ++i) a_frag[i] = keep_or_zero(ok, xc[i]);
    }
#pragma unroll
    for (int i = 0; i < NS4; ++i) *reinterpret_cast<uint4*>(buf + (i * TILE + m) * LROW + st_c8 * 2) = a_frag[i];
  };

  // One super-chunk s of item `it`; (nx, ns, ngt) is the super-chunk whose
  // first token half is prefetched. Issue order: B fragments of the MFMA phase,
  // the second token half, then (after the first half is computed) the
  // prefetch, so waiting for the first half or for the B fragments never waits
  // for loads issued later.
  uint4 xA[NS4], xB[NS4], fA = make_uint4(0, 0, 0, 0), fB = make_uint4(0, 0, 0, 0);
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  // MFMA phase of super-chunk s from the tile in `buf`, B fragments pf.
  auto mfma_phase = [&](const Item& it, int64_t s, const unsigned char* buf, const uint4 (&pf)[NS4][NB])
                        __attribute__((always_inline)) {
    const int64_t cg = s * SC + wave * 32;
    // With POST, rows past T and channels past C hold values computed from
    // clamped loads (zeroing them before the store would turn the store into a
    // branch): their A fragments are replaced by zeros here. Without POST the
    // tile already holds zeros there. Either way a group past C adds nothing
    // against its clamped, valid B address.
    const bool ch_ok = cg + q * 8 < C;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const bool a_ok = ch_ok && ((int64_t)it.tile * TILE + tb * TOK + tau < T);
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        uint4 af = *reinterpret_cast<const uint4*>(buf + (i * TILE + tb * TOK + tau) * LROW + (wave * 32 + q * 8) * 2);
        if (POST) af = keep_or_zero(a_ok, af);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(pf[i][b]), acc[tb][b], 0, 0, 0);
        // A times its own transpose: the diagonal accumulates each token's sum of squares.
        gram[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(af), gram[tb], 0, 0, 0);
      }
    }
    // The next super-chunk writes the other buffer; the one after it writes this
    // buffer only after passing the next barrier, i.e. after these reads.
  };

  auto body = [&](const Item& it, int64_t s, const int* gt, const Item& nx, int64_t ns, const int* ngt,
                  unsigned char* buf, const float* cf, __amdgpu_buffer_rsrc_t yres) __attribute__((always_inline)) {
    const int64_t cg = s * SC + wave * 32;
    const int64_t cgc = cg < C ? cg : C - 32;
    const int64_t prow0 = (MODE == ROWS_GROUPS ? 4 * it.g : 0) * C;  // phi row of stream 0 of the item
    uint4 pf[NS4][NB];
#pragma unroll
    for (int i = 0; i < NS4; ++i) {
      const uint4* pb = reinterpret_cast<const uint4*>(A.phi_p) + ((prow0 + i * C + cgc) / 8 + q) * NCP + tau;
#pragma unroll
      for (int b = 0; b < NB; ++b) pf[i][b] = pb[b * 16];
    }
    load_half(it, s, gt, H1{}, xB, fB);
    stream_half(it, s, H0{}, xA, fA, buf, cf, yres);
    load_half(nx, ns, ngt, H0{}, xA, fA);
    stream_half(it, s, H1{}, xB, fB, buf, cf, yres);
    __syncthreads();
    mfma_phase(it, s, buf, pf);
  };

  // Without POST the streaming work is only the copy into LDS, so more of the
  // state can be in flight: a queue of 4 token halves, filled 2 super-chunks
  // ahead. Half h of an item (h = 2 j + p) uses queue slot h mod 4 (an item
  // has 2 SPI halves, a multiple of 4, so the slot is a compile-time constant);
  // once half h is in LDS its slot is refilled with half h + 4, which for the
  // last 4 halves is one of the next item's first 4.
  constexpr bool DEEP = !POST && !(MODE == ROWS_GATHER && NB >= 4);  // (the latter has no registers left)
  constexpr bool RED2 = (SWAVE * TILE * (NCP + 1) + SWAVE * TILE) * 4 > LBUF;
  static_assert((SWAVE * TILE * (NCP + 1) + SWAVE * TILE) * 4 <= 2 * LBUF, "reduction buffer");
  static_assert(2 * SPI % 4 == 0, "queue slots of the deep prefetch");
  uint4 xq[DEEP ? 4 : 1][NS4];
  // DEEP: the B fragments of the super-chunk being multiplied. Each stream's are
  // replaced by the next super-chunk's as soon as its MFMAs have issued, so that
  // load has a whole super-chunk to arrive (the copy into LDS is too short to
  // hide an L2 round trip).
  uint4 pfq[DEEP ? NS4 : 1][NB];
  auto load_pf = [&](const Item& it2, int64_t s2, int i, uint4 (&dst)[NB]) __attribute__((always_inline)) {
    const int64_t cg = s2 * SC + wave * 32;
    const int64_t cgc = cg < C ? cg : C - 32;
    const int64_t prow0 = (MODE == ROWS_GROUPS ? 4 * it2.g : 0) * C;
    const uint4* pb = reinterpret_cast<const uint4*>(A.phi_p) + ((prow0 + i * C + cgc) / 8 + q) * NCP + tau;
#pragma unroll
    for (int b = 0; b < NB; ++b) dst[b] = pb[b * 16];
  };
  // Without POST the tile holds zeros for rows past T and channels past C.
  auto mfma_phase_deep = [&](const unsigned char* buf, const Item& nit, int64_t ns) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NS4; ++i) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const uint4 af =
            *reinterpret_cast<const uint4*>(buf + (i * TILE + tb * TOK + tau) * LROW + (wave * 32 + q * 8) * 2);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(pfq[i][b]), acc[tb][b], 0, 0, 0);
        gram[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(af), gram[tb], 0, 0, 0);
      }
      if constexpr (DEEP) load_pf(nit, ns, i, pfq[i]);
    }
  };
  auto body_deep = [&](const Item& it, auto J, const int* gt, const Item& nx, const int* ngt, unsigned char* buf)
                       __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int h0 = 2 * j, h1 = 2 * j + 1;
    constexpr int q0 = DEEP ? h0 % 4 : 0, q1 = DEEP ? h1 % 4 : 0;
    const int64_t s = it.s0 + j;
    uint4 fz = make_uint4(0, 0, 0, 0);
    const __amdgpu_buffer_rsrc_t nores = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0u, BUF_DW3);
    stream_half(it, s, H0{}, xq[q0], fz, buf, nullptr, nores);
    if constexpr (h0 + 4 < 2 * SPI) load_half(it, it.s0 + (h0 + 4) / 2, gt, H0{}, xq[q0], fz);
    else load_half(nx, nx.s0 + (h0 + 4 - 2 * SPI) / 2, ngt, H0{}, xq[q0], fz);
    stream_half(it, s, H1{}, xq[q1], fz, buf, nullptr, nores);
    if constexpr (h1 + 4 < 2 * SPI) load_half(it, it.s0 + (h1 + 4) / 2, gt, H1{}, xq[q1], fz);
    else load_half(nx, nx.s0 + (h1 + 4 - 2 * SPI) / 2, ngt, H1{}, xq[q1], fz);
    __syncthreads();
    // the next super-chunk: this item's next one, or the next item's first
    if constexpr (j + 1 < SPI) mfma_phase_deep(buf, it, it.s0 + j + 1);
    else mfma_phase_deep(buf, nx, nx.s0);
  };

  int item = (int)blockIdx.x;
  Item it = item_of(item);
  if (POST) {
    coef[tid] = coef_val(it.tile, tid);
    if (tid + STHR < NCOEF) coef[tid + STHR] = coef_val(it.tile, tid + STHR);
  }
  if (MODE == ROWS_GATHER) {
    const int v = gidx_val(it.tile);
    if (tid < TILE * 4) gtab[tid] = v;
  }
  if (POST || MODE == ROWS_GATHER) __syncthreads();
  if constexpr (DEEP) {
    uint4 fz = make_uint4(0, 0, 0, 0);
    load_half(it, it.s0, gtab, H0{}, xq[0], fz);
    load_half(it, it.s0, gtab, H1{}, xq[1], fz);
    load_half(it, it.s0 + 1, gtab, H0{}, xq[2], fz);
    load_half(it, it.s0 + 1, gtab, H1{}, xq[3], fz);
#pragma unroll
    for (int i = 0; i < NS4; ++i) load_pf(it, it.s0, i, pfq[i]);
  } else {
    load_half(it, it.s0, gtab, H0{}, xA, fA);
  }
  // the partial sums this thread reduced for the previous item (pitem; -1: none)
  float pend[PG::NPEND];
#pragma unroll
  for (int u = 0; u < PG::NPEND; ++u) pend[u] = 0.f;
  int pitem = -1;
  auto store_pending = [&]() __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)pitem * (uint32_t)(PG::PART * 4);
#pragma unroll
    for (int u = 0; u < PG::NPEND; ++u) {
      const int o = tid + u * STHR;
      const uint32_t off = pitem >= 0 && o < PG::PART ? base + (uint32_t)o * 4 : OOB;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend[u]), pres, off, 0, 0);
    }
  };
  int step = 0;
  for (int k = 0; k < nk; ++k) {
    // the next item of this workgroup (this one again after the last: its first
    // super-chunk is then prefetched for nothing)
    const int nitem_k = k + 1 < nk ? item + G : item;
    const Item nx = item_of(nitem_k);
    const float* cf = coef + (k & 1) * NCOEF;
    const int* gt = gtab + (k & 1) * (TILE * 4);
    const int* ngt = gtab + ((k + 1) & 1) * (TILE * 4);
    const int64_t nrow = (T - (int64_t)it.tile * TILE) < TILE ? (T - (int64_t)it.tile * TILE) : TILE;
    const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
        POST ? A.Y + (int64_t)it.tile * TILE * (NS4 * C) : nullptr, 0, POST ? (uint32_t)(nrow * NS4 * C * 2) : 0u,
        BUF_DW3);
    float cn0 = 0.f, cn1 = 0.f;
    // the next item's stream indices: the deep prefetch reads them from the
    // third super-chunk on, the other one in the last super-chunk
    int gn = 0;
    if (DEEP && MODE == ROWS_GATHER) gn = gidx_val(nx.tile);
    // SPI super-chunks, unrolled (past the last super-chunk of C they only add
    // zeros): straight-line code keeps the compiler's wait counts exact.
    auto tail = [&](int j) __attribute__((always_inline)) {
      if (j == 0) {
        // after the first prefetch: the previous item's partial sums and the
        // next item's coefficients and stream indices
        store_pending();
        if (POST) {
          cn0 = coef_val(nx.tile, tid);
          cn1 = coef_val(nx.tile, cidx1);
        }
        if (!DEEP && MODE == ROWS_GATHER) gn = gidx_val(nx.tile);
      }
      if (j == (DEEP ? 0 : 1) && MODE == ROWS_GATHER) {
        // visible after the next barrier, before the first read for the next
        // item; this item's reads of that buffer ended in the previous item
        if (tid < TILE * 4) gtab[((k + 1) & 1) * (TILE * 4) + tid] = gn;
      }
    };
    if constexpr (DEEP) {
      static_for<SPI>([&](auto J) __attribute__((always_inline)) {
        body_deep(it, J, gt, nx, ngt, lds + ((step + decltype(J)::value) & 1) * LBUF);
        tail(decltype(J)::value);
      });
    } else {
#pragma unroll
      for (int j = 0; j < SPI; ++j) {
        const bool last = j + 1 == SPI;
        body(it, it.s0 + j, gt, last ? nx : it, last ? nx.s0 : it.s0 + j + 1, last ? ngt : gt,
             lds + ((step + j) & 1) * LBUF, cf, yres);
        tail(j);
      }
    }
    step += SPI;
    // ---- item end: cross-wave reduction into this thread's partial sums,
    // through the buffer the last super-chunk's MFMA phase read (through both
    // buffers when the partials of more than 32 columns do not fit one)
    __syncthreads();
    float* red = reinterpret_cast<float*>(RED2 ? lds : lds + ((step - 1) & 1) * LBUF);  // [SWAVE][TILE][NCP + 1]
    float* ssr = red + SWAVE * TILE * (NCP + 1);                                        // [SWAVE][TILE]
    // lane holds D[m = q*4 + e][n = tau] of each block b, for token block tb
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          red[(wave * TILE + tb * TOK + q * 4 + e) * (NCP + 1) + b * 16 + tau] = acc[tb][b][e];
    // the diagonal m == n of gram[tb] sits in the lane with tau == q*4 + e
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (tau == q * 4 + e) ssr[wave * TILE + tb * TOK + tau] = gram[tb][e];
    if (POST) {
      float* cn = coef + ((k + 1) & 1) * NCOEF;
      cn[tid] = cn0;
      if (tid + STHR < NCOEF) cn[tid + STHR] = cn1;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      gram[tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();
    auto reduce = [&](int o) __attribute__((always_inline)) {
      const int m = o / PG::PROW, col = o - m * PG::PROW;
      float sum = 0.f;
      if (col < PG::NCOLP) {
#pragma unroll
        for (int w = 0; w < SWAVE; ++w)
          sum += red[(w * TILE + m) * (NCP + 1) + col] + red[(w * TILE + m) * (NCP + 1) + PG::NCOLP + col];
      } else {
#pragma unroll
        for (int w = 0; w < SWAVE; ++w) sum += ssr[w * TILE + m];
      }
      return sum;
    };
#pragma unroll
    for (int u = 0; u < PG::NPEND; ++u) {
      const int o = tid + u * STHR;
      pend[u] = reduce(o < PG::PART ? o : tid);
    }
    if constexpr (RED2) __syncthreads();  // the next item's first half is written into buffer 0
    pitem = item;
    item = nitem_k;
    it = nx;
  }
  store_pending();
}

// ---------------------------------------------------------- 64-token items
// Projection only (no post/res write) with items of W_TOK = 64 tokens: each
// packed-phi fragment taken from L2 serves 64 tokens instead of 32, half the L2
// traffic per byte of state (measured: with every wave loading the same phi the
// 32-token kernel runs 22% faster, so that traffic, not the MFMA work, is what
// costs). Item = 64 tokens x a group of 4 streams x W_SPI super-chunks of W_SC
// = 128 channels (1024 channels), numbered tile-major as in mhc_split_kernel;
// per-item partials [64][NB*8 + 1] in float, added by the finish kernels.
//  * streaming phase: thread (token tid >> 4, and + 32 for the second half; 8
//    channels at (tid & 15) * 8) loads its 16-byte pieces of the 4 streams: 16
//    consecutive lanes read 256 contiguous bytes of a stream row;
//  * MFMA phase: wave w takes the 32-channel group w & 3 of the super-chunk for
//    streams 2 (w >> 2) and 2 (w >> 2) + 1 and all 4 token blocks.
// Four token halves (two super-chunks) are in flight; each stream's phi
// fragments for the next super-chunk load right after its MFMAs.
constexpr int W_TOK = 64;
constexpr int W_SC = 128;
constexpr int W_SPI = 8;
constexpr int W_LROW = W_SC * 2 + 16;         // bytes per (stream, token) row in LDS, padded
constexpr int W_LBUF = NS4 * W_TOK * W_LROW;  // bytes per LDS buffer

// With DH, each streaming thread also takes its 16-byte piece of dF_in at the
// same (token, channels) and adds <dF_in, x_i> over its 8 channels for the
// group's 4 streams; at the item end the 16 lanes of a token are summed (DPP)
// and the 4 sums go to the partial's extra columns (the gradient of the pre
// map's input in the xHC backward, from the same read of the state).
//
// When NB is even the hi and lo halves of the packed columns fall in separate
// 16-column blocks (hi blocks 0 .. NB/2 - 1, lo blocks NB/2 .. NB - 1), and each
// hi block and its lo block accumulate into one set of registers (the two
// products are added in float32 anyway): NB/2 accumulator sets per token block
// instead of NB, which is what lets 32 columns (NB = 4) run on 64-token items.
//
// QD token halves are in flight (4: two super-chunks ahead; 2: one, for the
// widest column counts, whose accumulators and phi fragments need the registers).
// NTG (ROWS_GATHER): nontemporal loads of the gathered rows.
template <int NB, int MODE, bool DH = false, bool SH = false, int QD = 4,
          bool NTG = false>  // SH: hi and lo share accumulators
__global__ __launch_bounds__(STHR) void proj_wide_kernel(SplitArgs A) {
  static_assert(!SH || NB % 2 == 0, "shared accumulators pair hi block b with lo block b + NB / 2");
  static_assert(QD == 2 || QD == 4, "token halves in flight");
  constexpr bool DENSE = MODE == ROWS_DENSE, PAIRS = MODE == ROWS_PAIRS, GATH = MODE == ROWS_GATHER;
  static_assert(!(DH && (DENSE || PAIRS || GATH)), "the dF_in sums are for the stream-group and contiguous rows");
  // DENSE: the 4 stream groups of one 128-channel super-chunk are consecutive
  // steps, so an item covers W_SPI / 4 super-chunks of every group
  constexpr int NGD = DENSE ? 4 : 1;
  static_assert(W_SPI % NGD == 0, "steps per item");
  // The state and phi read through buffer resources with per-step scalar
  // offsets (one per-thread offset for every step), where 64-bit addresses per
  // step and stream would not fit the registers: the dense rows, whose steps
  // change stream group, and the widest stream-group passes (NB >= 6, the
  // xHC-Flash block entry). The host keeps a tile's rows under 4 GiB.
  constexpr bool BUFL = DENSE || (MODE == ROWS_GROUPS && !DH && NB >= 6);
  constexpr int NA = SH ? NB / 2 : NB;   // accumulator sets per token block
  static_assert(NA <= 5, "4 token blocks x more accumulator sets exceed the registers");
  using PG = PartGeom<NB, W_TOK, DH ? NS4 : 0>;
  constexpr int NCP = PG::NCP;
  constexpr int RS = NA * 16 + 1;  // floats per (wave, token) row of the reduction buffer
  // the item-end reduction takes TPR tokens per round through one LDS buffer
  constexpr int TPR = SWAVE * 32 * RS * 4 + SWAVE * 32 * 4 + 32 * NS4 * 4 <= W_LBUF ? 32 : 16;
  constexpr int NR = W_TOK / TPR;                            // rounds
  constexpr int NPH = (TPR * PG::PROW + STHR - 1) / STHR;   // partial floats per thread per round
  static_assert(SWAVE * TPR * RS * 4 + SWAVE * TPR * 4 + TPR * NS4 * 4 <= W_LBUF, "reduction buffer");
  static_assert(!(DH || DENSE) || TPR == 32, "the dF_in sums and DENSE's sums of squares are kept per 32-token half");
  const uint16_t* X = A.X;
  const int64_t T = A.T, C = A.C;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * W_LBUF];
  // Per-token tables of the item being streamed and of the next item: PAIRS, the
  // pair tokens; DENSE, the tokens' h_pre (htab) and the mask of their active
  // streams (ptab); GATH, the tokens' 4 stream indices (ptab, 4 per token)
  constexpr bool TAB = PAIRS || DENSE || GATH;
  constexpr int TABW = GATH ? 4 * W_TOK : W_TOK;  // ints per table
  __shared__ __attribute__((aligned(16))) int ptab[TAB ? 2 * TABW : 1];
  __shared__ __attribute__((aligned(16))) float htab[DENSE ? 2 * W_TOK * 16 : 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int st_tok = tid >> 4;
  const int st_c8 = (tid & 15) * 8;
  const int tau = lane & 15;
  const int q = lane >> 4;
  const int cgw = wave & 3, sp = wave >> 2;
  const int G = (int)gridDim.x;
  // Items of this workgroup: blockIdx.x, + G, ... (>= 1); PAIRS: the items are
  // split into 8 contiguous ranges, one per XCD (workgroups go to the XCDs in
  // turn, workgroup b to XCD b mod 8), so each XCD's L2 holds the phi rows of the
  // 2-3 buckets its range covers instead of every stream's
  constexpr int NXCD = 8;
  const bool xcd_map = PAIRS && G % NXCD == 0;
  const int xs = (int)blockIdx.x % NXCD, xslot = (int)blockIdx.x / NXCD, GX = G / NXCD;
  const int x_lo = xcd_map ? (int)((int64_t)xs * A.nitem / NXCD) : 0;
  const int x_hi = xcd_map ? (int)((int64_t)(xs + 1) * A.nitem / NXCD) : A.nitem;
  const int stride = xcd_map ? GX : G;
  const int first_item = xcd_map ? x_lo + xslot : (int)blockIdx.x;
  const int nk = first_item < x_hi ? (x_hi - first_item + stride - 1) / stride : 0;
  if (nk == 0) return;  // (uniform over the workgroup, before any barrier)
  // items per tile (DENSE: 256-channel steps of all groups, as many as the
  // group x 1024-channel items of the other modes)
  const int per_tile = A.NG * A.S;

  floatx4_t acc[4][NA], gram[4];
#pragma unroll
  for (int tb = 0; tb < 4; ++tb) {
    gram[tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NA; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }
  const __amdgpu_buffer_rsrc_t pres =
      __builtin_amdgcn_make_buffer_rsrc(A.part, 0, (uint32_t)((int64_t)A.nitem * PG::PART * 4), BUF_DW3);

  // g: the stream group (GROUPS; DENSE steps set their own), or the bucket's
  // stream (PAIRS)
  struct Item {
    int tile, g;
    int64_t s0;
  };
  auto item_of = [&](int item) __attribute__((always_inline)) {
    const int tile = item / per_tile;
    const int r = item - tile * per_tile;
    if constexpr (DENSE) return Item{tile, 0, (int64_t)r * (W_SPI / NGD)};
    if constexpr (PAIRS) {
      // the bucket holding pair tile `tile` (tiles past the last bucket: the last
      // stream, their pairs are all padding)
      int b = 0;
      for (int z = 1; z < A.nstreams; ++z) b = A.tile_off[z] <= tile ? z : b;
      return Item{tile, b, (int64_t)r * W_SPI};
    }
    if constexpr (MODE == ROWS_GROUPS && DH) {
      // Blocks of 2 tiles with the stream group as the stride-2S digit: with S = 4
      // slices the 4 groups of one (tile, slice) are 8 items apart, so they run on
      // one XCD in the same round and read that slice of dF_in through one L2
      // (the last block of an odd tile count keeps the tile-major order)
      const int blk = 2 * per_tile;
      const int pb = item / blk, rb = item - pb * blk;
      if (2 * pb + 1 < (A.nitem / per_tile)) {
        const int g = rb / (2 * A.S), rest = rb - g * 2 * A.S;
        const int half = rest / A.S;
        return Item{2 * pb + half, g, (int64_t)(rest - half * A.S) * W_SPI};
      }
    }
    const int g = r / A.S;
    return Item{tile, g, (int64_t)(r - g * A.S) * W_SPI};
  };
  // where an item's partials go: its tile-major index, the order the finish
  // kernels add them in (the schedule order differs for the dF_in-sum mode)
  auto part_index = [&](int item, const Item& it) __attribute__((always_inline)) {
    if constexpr (MODE == ROWS_GROUPS && DH) return it.tile * per_tile + it.g * A.S + (int)(it.s0 / W_SPI);
    return item;
  };
  // first stream of an item's rows at stream group g (GROUPS, DENSE)
  auto stream0 = [&](int g) __attribute__((always_inline)) { return MODE == ROWS_GROUPS || DENSE ? 4 * g : 0; };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  // Loads are unconditional (clamped rows and channels), as in mhc_split_kernel.
  // Step js of an item: super-chunk s0 + js / NGD, stream group js % NGD (DENSE);
  // pt: the item's PAIRS table.
  auto load_half = [&](const Item& it, int js, const int* pt, auto P, uint4 (&xv)[NS4], uint4& dv)
                       __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int64_t s = it.s0 + js / NGD;
    const int g = DENSE ? js % NGD : it.g;
    if constexpr (BUFL) {
      // Buffer loads over the item's tile of token rows (rows past T read as
      // zeros; channels past C, the next row's, are zeroed when streamed).
      const int64_t r0 = (int64_t)it.tile * W_TOK;
      const int64_t nrow = T - r0 < W_TOK ? T - r0 : W_TOK;
      const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(X) + r0 * A.rowstride, 0, (uint32_t)(nrow * A.rowstride * 2), BUF_DW3);
      const uint32_t vo = (uint32_t)(((int64_t)(st_tok + 32 * p) * A.rowstride + st_c8) * 2);
      const uint32_t so = (uint32_t)(((int64_t)stream0(g) * C + s * W_SC) * 2);
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(xrs, vo, so + (uint32_t)(i * C * 2), 2);
        xv[i] = make_uint4(v.x, v.y, v.z, v.w);
      }
      return;
    }
    int64_t t;
    if constexpr (PAIRS) {
      const int v = pt[st_tok + 32 * p];
      t = v < 0 ? 0 : (v >= T ? T - 1 : v);
    } else {
      t = (int64_t)it.tile * W_TOK + st_tok + 32 * p;
      t = t < T ? t : T - 1;
    }
    const int64_t c = s * W_SC + st_c8;
    const int64_t cc = c < C ? c : C - 8;
    if constexpr (GATH) {
      // the token's 4 streams from the table (clamped into the row); ordinary
      // (cache-allocating) loads unless NTG: the mix pass that follows reads
      // these rows again, newest first, and finds part of them in the
      // last-level cache, which pays where it reads little else (K = 1)
      const int4 z4 = *reinterpret_cast<const int4*>(pt + (st_tok + 32 * p) * 4);
      const int zs[NS4] = {z4.x, z4.y, z4.z, z4.w};
      const uint16_t* xr = X + t * A.rowstride + cc;
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        const int z = zs[i] < 0 ? 0 : (zs[i] >= A.nstreams ? A.nstreams - 1 : zs[i]);
        if constexpr (NTG) xv[i] = ld_stream(xr + (int64_t)z * C);
        else xv[i] = *reinterpret_cast<const uint4*>(xr + (int64_t)z * C);
      }
      return;
    }
    const uint16_t* xg = X + t * A.rowstride + cc + (PAIRS ? (int64_t)g * A.sq : (int64_t)stream0(g) * C);
#pragma unroll
    for (int i = 0; i < NS4; ++i) xv[i] = ld_stream(xg + i * C);
    if constexpr (DH) dv = ld_stream(A.dF + t * C + cc);
  };
  float dh[2][NS4];  // DH: this thread's <dF_in, x_i> of the item, per token half
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int i = 0; i < NS4; ++i) dh[r][i] = 0.f;
  // DENSE: the sum of squares of the rows kept in the projection, this thread's
  // channels of its token in each half (taken with F_in instead of on MFMA)
  float ssd[2] = {0.f, 0.f};
  float fin[2][8];  // DENSE: this thread's F_in of the current super-chunk, per token half
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) fin[r][e] = 0.f;
  // the tile in LDS holds zeros for rows past T and channels past C (PAIRS: and
  // for padding; pt is the item's table)
  auto stream_half = [&](const Item& it, int js, const int* pt, auto P, const uint4 (&xc)[NS4], const uint4& dc,
                         unsigned char* buf) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int m = st_tok + 32 * p;
    const int64_t s = it.s0 + js / NGD;
    const bool row_ok = PAIRS ? pt[m] >= 0 : ((int64_t)it.tile * W_TOK + m < T);
    const bool ok = row_ok && (s * W_SC + st_c8 < C);
    const uint4 dz = keep_or_zero(ok, dc);
#pragma unroll
    for (int i = 0; i < NS4; ++i) {
      const uint4 xz = keep_or_zero(ok, xc[i]);
      *reinterpret_cast<uint4*>(buf + (i * W_TOK + m) * W_LROW + st_c8 * 2) = xz;
      if constexpr (DH) {  // bf16 pairs multiplied into the float32 sum (v_dot2_f32_bf16)
        float a = dh[p][i];
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xz.x), as_bf16x2(dz.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xz.y), as_bf16x2(dz.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xz.z), as_bf16x2(dz.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xz.w), as_bf16x2(dz.w), a, false);
        dh[p][i] = a;
      }
    }
  };
  // DENSE, once the step's tile is in LDS: this thread's F_in pieces (the rows
  // it streamed, read back from the tile, every row in stream order as
  // pre_wide_kernel adds them); after the last group of a super-chunk they are
  // complete and stored. (Adding them from the loaded registers while the
  // queue refills holds enough of them at once to spill.)
  auto dense_read = [&](const Item& it, int js, const int* pt, const float* ht, const unsigned char* buf,
                        __amdgpu_buffer_rsrc_t frs) __attribute__((always_inline)) {
    const int64_t s = it.s0 + js / NGD;
    const int g = js % NGD;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int m = st_tok + 32 * p;
      const float4 hc = *reinterpret_cast<const float4*>(ht + m * 16 + 4 * g);
      const float hw[4] = {hc.x, hc.y, hc.z, hc.w};
      const int amask = pt[m] >> (4 * g);
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        const uint4 xr = *reinterpret_cast<const uint4*>(buf + (i * W_TOK + m) * W_LROW + st_c8 * 2);
        float xv[8];
        unpack8(xr, xv);
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          fin[p][e] += hw[i] * xv[e];
          sq += xv[e] * xv[e];
        }
        ssd[p] += (amask >> i) & 1 ? 0.f : sq;
      }
      if (g == NGD - 1) {  // the last group of the super-chunk: these 8 channels are complete
        const int64_t c = s * W_SC + st_c8;
        const uint32_t off = c < C ? (uint32_t)(((int64_t)m * C + c) * 2) : OOB;
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pack_bf2_hw(fin[p][0], fin[p][1]), pack_bf2_hw(fin[p][2], fin[p][3]),
                                                       pack_bf2_hw(fin[p][4], fin[p][5]), pack_bf2_hw(fin[p][6], fin[p][7])},
                                               frs, off, 0, 0);
#pragma unroll
        for (int e = 0; e < 8; ++e) fin[p][e] = 0.f;
      }
    }
  };
  uint4 xq[QD][NS4];
  uint4 dq[QD];  // DH: the dF_in pieces beside xq
  uint4 pfq[2][NB];
  // BUFL: the phi fragments through a buffer resource as well, the wave's row
  // offset in the scalar offset (its stream and channel group are wave-uniform)
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A.phi_p), 0, BUFL ? (uint32_t)(A.rowstride / 8 * NCP * 16) : 0u, BUF_DW3);
  auto load_pf = [&](const Item& it2, int js2, int si, uint4 (&dst)[NB]) __attribute__((always_inline)) {
    const int64_t s2 = it2.s0 + js2 / NGD;
    const int g2 = DENSE ? js2 % NGD : it2.g;
    if constexpr (BUFL) {
      // (a group past C reads the next stream's rows, or zeros past the end, and
      // meets zero A fragments)
      const int64_t cg = s2 * W_SC + (wu & 3) * 32;
      const int64_t prow0 = (int64_t)(stream0(g2) + 2 * (wu >> 2) + si) * C;
      const uint32_t so = (uint32_t)((prow0 + cg) / 8 * NCP * 16);
      const uint32_t vo = (uint32_t)((q * NCP + tau) * 16);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(prs, vo + (uint32_t)(b * 256), so, 0);
        dst[b] = make_uint4(v.x, v.y, v.z, v.w);
      }
      return;
    }
    const int64_t cg = s2 * W_SC + cgw * 32;
    const int64_t cgc = cg < C ? cg : C - 32;
    const int64_t prow0 = PAIRS ? (int64_t)g2 * A.sq + (int64_t)(2 * sp + si) * C
                                : (int64_t)(stream0(g2) + 2 * sp + si) * C;
    const uint4* pb = reinterpret_cast<const uint4*>(A.phi_p) + ((prow0 + cgc) / 8 + q) * NCP + tau;
#pragma unroll
    for (int b = 0; b < NB; ++b) dst[b] = pb[b * 16];
  };
  // DENSE: the tile holds every row; the rows of the active streams (bit of the
  // token's mask in pt) enter the MFMAs as zeros
  auto mfma_phase = [&](const unsigned char* buf, const Item& nit, int njs, int g, const int* pt)
                        __attribute__((always_inline)) {
#pragma unroll
    for (int si = 0; si < 2; ++si) {
      const int stream = 2 * sp + si;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        uint4 af = *reinterpret_cast<const uint4*>(buf + (stream * W_TOK + tb * TOK + tau) * W_LROW +
                                                   (cgw * 32 + q * 8) * 2);
        if constexpr (DENSE) af = keep_or_zero(!((pt[tb * TOK + tau] >> (4 * g + stream)) & 1), af);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[tb][b % NA] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(pfq[si][b]), acc[tb][b % NA], 0, 0, 0);
        if constexpr (!DENSE)
          gram[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(af), gram[tb], 0, 0, 0);
      }
      load_pf(nit, njs, si, pfq[si]);
    }
  };
  // Step j of item `it`: half h (= 2j + p) uses queue slot h mod QD and is
  // refilled with half h + QD (for the last QD halves: the next item's first QD).
  static_assert(2 * W_SPI % QD == 0, "queue slots");
  auto body = [&](const Item& it, auto J, const int* pt, const float* ht, const Item& nx, const int* npt,
                  unsigned char* buf, __amdgpu_buffer_rsrc_t frs) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;
    constexpr int h0 = 2 * j, h1 = 2 * j + 1;
    constexpr int q0 = h0 % QD, q1 = h1 % QD;
    stream_half(it, j, pt, H0{}, xq[q0], dq[q0], buf);
    if constexpr (h0 + QD < 2 * W_SPI) load_half(it, (h0 + QD) / 2, pt, H0{}, xq[q0], dq[q0]);
    else load_half(nx, (h0 + QD - 2 * W_SPI) / 2, npt, H0{}, xq[q0], dq[q0]);
    stream_half(it, j, pt, H1{}, xq[q1], dq[q1], buf);
    if constexpr (h1 + QD < 2 * W_SPI) load_half(it, (h1 + QD) / 2, pt, H1{}, xq[q1], dq[q1]);
    else load_half(nx, (h1 + QD - 2 * W_SPI) / 2, npt, H1{}, xq[q1], dq[q1]);
    __syncthreads();
    if constexpr (DENSE) dense_read(it, j, pt, ht, buf, frs);
    if constexpr (j + 1 < W_SPI) mfma_phase(buf, it, j + 1, j % NGD, pt);
    else mfma_phase(buf, nx, 0, j % NGD, pt);
  };

  // The tables of an item: loaded into registers (tab_load), then written to
  // LDS buffer b (tab_store) once they have arrived.
  int tv_i = 0;
  float2 tv_h = make_float2(0.f, 0.f);
  int4 tv_x = make_int4(0, 0, 0, 0);
  auto tab_load = [&](const Item& it2) __attribute__((always_inline)) {
    if constexpr (PAIRS) tv_i = tid < W_TOK ? A.ptok[(int64_t)it2.tile * W_TOK + tid] : 0;
    if constexpr (GATH) {
      if (tid < 4 * W_TOK) {
        int64_t t2 = (int64_t)it2.tile * W_TOK + (tid >> 2);
        t2 = t2 < T ? t2 : T - 1;
        tv_i = A.idx[t2 * A.kidx + (tid & 3)];
      }
    }
    if constexpr (DENSE) {
      int64_t t = (int64_t)it2.tile * W_TOK + (tid >> 3);
      t = t < T ? t : T - 1;
      tv_h = *reinterpret_cast<const float2*>(A.hd + t * 16 + (tid & 7) * 2);
      if (tid < W_TOK) {
        int64_t t2 = (int64_t)it2.tile * W_TOK + tid;
        t2 = t2 < T ? t2 : T - 1;
        tv_x = *reinterpret_cast<const int4*>(A.idx + t2 * 4);
      }
    }
  };
  auto tab_store = [&](int b) __attribute__((always_inline)) {
    if constexpr (PAIRS) {
      if (tid < W_TOK) ptab[b * W_TOK + tid] = tv_i;
    }
    if constexpr (GATH) {
      if (tid < 4 * W_TOK) ptab[b * TABW + tid] = tv_i;
    }
    if constexpr (DENSE) {
      *reinterpret_cast<float2*>(htab + b * W_TOK * 16 + (tid >> 3) * 16 + (tid & 7) * 2) = tv_h;
      if (tid < W_TOK) {
        // bit z: stream z is active (indices outside [0, 16) mark nothing)
        auto bit = [](int z) { return z >= 0 && z < 16 ? 1 << z : 0; };
        ptab[b * W_TOK + tid] = bit(tv_x.x) | bit(tv_x.y) | bit(tv_x.z) | bit(tv_x.w);
      }
    }
  };

  int item = first_item;
  Item it = item_of(item);
  if constexpr (TAB) {
    tab_load(it);
    tab_store(0);
    __syncthreads();
  }
  load_half(it, 0, ptab, H0{}, xq[0], dq[0]);
  load_half(it, 0, ptab, H1{}, xq[1], dq[1]);
  if constexpr (QD == 4) {
    load_half(it, 1, ptab, H0{}, xq[2 % QD], dq[2 % QD]);
    load_half(it, 1, ptab, H1{}, xq[3 % QD], dq[3 % QD]);
  }
  load_pf(it, 0, 0, pfq[0]);
  load_pf(it, 0, 1, pfq[1]);
  // the partial sums this thread reduced for the previous item (pitem; -1: none):
  // pend[r][u] holds element tid + u * STHR of the item's token half r
  float pend[NR][NPH];
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int u = 0; u < NPH; ++u) pend[r][u] = 0.f;
  int pitem = -1;
  auto store_pending = [&]() __attribute__((always_inline)) {
    const uint32_t base = (uint32_t)pitem * (uint32_t)(PG::PART * 4);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int u = 0; u < NPH; ++u) {
        const int o = tid + u * STHR;
        const uint32_t off = pitem >= 0 && o < TPR * PG::PROW ? base + (uint32_t)(r * TPR * PG::PROW + o) * 4 : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pend[r][u]), pres, off, 0, 0);
      }
  };
  int step = 0;
  for (int k = 0; k < nk; ++k) {
    const int nitem_k = k + 1 < nk ? item + stride : item;
    const Item nx = item_of(nitem_k);
    const int* pt = ptab + (TAB ? (k & 1) * TABW : 0);
    const int* npt = ptab + (TAB ? ((k + 1) & 1) * TABW : 0);
    const float* ht = htab + (DENSE ? (k & 1) * W_TOK * 16 : 0);
    // The next item's tables: loaded now, written to the other buffer after the
    // second step's barrier (that buffer's last reads, by the previous item, came
    // before the first), so the next item's first prefetch (step W_SPI - QD / 2)
    // and first streaming step find them.
    if constexpr (TAB) tab_load(nx);
    // DENSE: F_in rows of this item's tile
    __amdgpu_buffer_rsrc_t frs = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0u, BUF_DW3);
    if constexpr (DENSE) {
      const int64_t r0 = (int64_t)it.tile * W_TOK;
      const int64_t nrow = T - r0 < W_TOK ? T - r0 : W_TOK;
      frs = __builtin_amdgcn_make_buffer_rsrc(A.Fd + r0 * C, 0, (uint32_t)(nrow * C * 2), BUF_DW3);
    }
    static_for<W_SPI>([&](auto J) __attribute__((always_inline)) {
      body(it, J, pt, ht, nx, npt, lds + ((step + decltype(J)::value) & 1) * W_LBUF, frs);
      if constexpr (decltype(J)::value == 0) store_pending();
      if constexpr (decltype(J)::value == 1 && TAB) tab_store((k + 1) & 1);
    });
    step += W_SPI;
    // item end: the 8 waves' sums, TPR tokens (TPR / 16 token blocks) per round,
    // through the buffer the last MFMA phase read
    float* red = reinterpret_cast<float*>(lds + ((step - 1) & 1) * W_LBUF);  // [SWAVE][TPR][RS]
    float* ssr = red + SWAVE * TPR * RS;                                      // [SWAVE][TPR]
    float* dhr = ssr + SWAVE * TPR;                                           // DH: [32][NS4]
    if constexpr (DH) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < NS4; ++i) dh[r][i] = row16_sum(dh[r][i]);
    }
    if constexpr (DENSE) {
      ssd[0] = row16_sum(ssd[0]);
      ssd[1] = row16_sum(ssd[1]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      __syncthreads();
      if constexpr (DH) {
        if ((tid & 15) == 0) {
#pragma unroll
          for (int i = 0; i < NS4; ++i) dhr[st_tok * NS4 + i] = dh[r][i];
        }
      }
      if constexpr (DENSE) {  // (TPR == 32: round r is token half r)
        if ((tid & 15) == 0) dhr[st_tok] = ssd[r];
      }
#pragma unroll
      for (int tbb = 0; tbb < TPR / TOK; ++tbb) {
        const int tb = (TPR / TOK) * r + tbb;
#pragma unroll
        for (int b = 0; b < NA; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            red[(wave * TPR + tbb * TOK + q * 4 + e) * RS + b * 16 + tau] = acc[tb][b][e];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (tau == q * 4 + e) ssr[wave * TPR + tbb * TOK + tau] = gram[tb][e];
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < NPH; ++u) {
        int o = tid + u * STHR;
        o = o < TPR * PG::PROW ? o : tid;
        const int m = o / PG::PROW, col = o - m * PG::PROW;
        float sum = 0.f;
        if (col < PG::NCOLP) {
#pragma unroll
          for (int w = 0; w < SWAVE; ++w) {
            if constexpr (SH) sum += red[(w * TPR + m) * RS + col];
            else sum += red[(w * TPR + m) * RS + col] + red[(w * TPR + m) * RS + PG::NCOLP + col];
          }
        } else if (col == PG::NCOLP) {
          if constexpr (DENSE) {
            sum = dhr[m];
          } else {
#pragma unroll
            for (int w = 0; w < SWAVE; ++w) sum += ssr[w * TPR + m];
          }
        } else {
          sum = dhr[m * NS4 + (col - PG::NCOLP - 1)];
        }
        pend[r][u] = sum;
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int i = 0; i < NS4; ++i) dh[r][i] = 0.f;
    ssd[0] = ssd[1] = 0.f;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      gram[tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < NA; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    pitem = part_index(item, it);
    item = nitem_k;
    it = nx;
  }
  store_pending();
}

// Partial sums of an item: W_TOK-token items (proj_wide_kernel) or TILE-token
// items (mhc_split_kernel); the finish kernels take the item size TT.

// 1 / r with r = sqrt(ss / 4C), the token's RMS over the flattened state
// (0 for an all-zero state), and the gate logit alpha * P / r + b: shared by
// every kernel that forms mHC gates, so they produce the same floats.
__device__ __forceinline__ float inv_rms4(float ss, int64_t C) {
  const float r = sqrtf(ss / (float)(NS4 * C));
  return (r > 0.f) ? 1.0f / r : 0.f;
}
__device__ __forceinline__ float gate_logit(float a, float p, float invr, float b) { return a * (p * invr) + b; }

// Coefficients of token tt (< T) from the partial projections ([mHC] Eq.
// 15-19), computed by the 16 lanes of one DPP row (lane e = tid & 15). Each lane
// adds the token's slices in slice order (the sum of squares, the h_res logit
// of entry e = i*4 + j, and for e < 8 the pre/post logit), then r = sqrt(ss /
// 4C), z = alpha * P / r + b, h_pre = sigmoid, h_post = 2 sigmoid, and
// Sinkhorn-Knopp on the 4x4 block held by the 16 lanes. Returns h_pre[e] in
// lanes e < 4; stores the coefficients when `store` (uniform over the row).
// TT: tokens per item of the partials.
template <int TT>
__device__ __forceinline__ float token_coeffs(const float* __restrict__ part, int64_t tt, int e, int64_t C, int S,
                                              const float* __restrict__ bias, Gate gate, int iters, bool store,
                                              float* __restrict__ h_pre_out, float* __restrict__ h_post_out,
                                              float* __restrict__ h_res_out) {
  using PG = PartGeom<3, TT>;
  const int64_t tile = tt / TT;
  const int m = (int)(tt - tile * TT);
  const float* base = part + tile * S * PG::PART + m * PG::PROW;
  float ss = 0.f, pr = 0.f, pe = 0.f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float* b = base + (int64_t)s * PG::PART;
    ss += b[PG::NCOLP];
    pr += b[8 + e];
    pe += b[e & 7];
  }
  const float invr = inv_rms4(ss, C);
  const float a = e < 4 ? gate.a_pre : gate.a_post;
  const float sg = sigmoid(gate_logit(a, pe, invr, bias[e & 7]));
  if (store && e < 8) {
    if (e < 4) {
      if (h_pre_out) h_pre_out[tt * 4 + e] = sg;
    } else {
      h_post_out[tt * 4 + (e - 4)] = 2.0f * sg;
    }
  }
  // h_res: the per-token max logit is subtracted before exp (a common factor of
  // M0, removed by the first normalisation). Cross-lane sums use DPP within the
  // 16-lane row: a column (fixed j) is lanes j, j+4, j+8, j+12, summed as
  // (M[e] + M[e+8]) + (M[e+4] + M[e+12]) by rotating 8 then 4, which gives the
  // same operands, hence the same float, in all four lanes; a row (fixed i) is
  // one quad, summed with the quad permutations xor 1, xor 2.
  const float z = gate_logit(gate.a_res, pr, invr, bias[8 + e]);
  float zm = fmaxf(z, dpp<DPP_QXOR1>(z));
  zm = fmaxf(zm, dpp<DPP_QXOR2>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR4>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR8>(zm));
  float M = expf(z - zm);
  for (int it = 0; it < iters; ++it) {
    float cs = M + dpp<DPP_ROR8>(M);  // column sum over i
    cs += dpp<DPP_ROR4>(cs);
    M = M / cs;
    float rs = M + dpp<DPP_QXOR1>(M);  // row sum over j
    rs += dpp<DPP_QXOR2>(rs);
    M = M / rs;
  }
  if (store) h_res_out[tt * 16 + e] = M;
  return sg;
}

// Coefficients only: 16 threads per token (every lane of a row takes part in
// the DPP exchanges; rows past T work on the last token and store nothing).
template <int TT>
__global__ __launch_bounds__(256) void coeffs_finish_kernel(const float* __restrict__ part, int64_t T, int64_t C,
                                                            int S, const float* __restrict__ bias, Gate gate,
                                                            int iters, float* __restrict__ h_pre_out,
                                                            float* __restrict__ h_post_out,
                                                            float* __restrict__ h_res_out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tt = g >> 4;
  token_coeffs<TT>(part, tt < T ? tt : T - 1, (int)(g & 15), C, S, bias, gate, iters, tt < T, h_pre_out, h_post_out,
                   h_res_out);
}

// ------------------------------------------------- mHC coefficient backward

// Backward of Eq. 15-19 for token tt, 16 lanes per token as in token_coeffs
// (lane e: h_res entry e = i*4 + j; lanes e < 8 also gate column e: pre for
// e < 4, post for 4 <= e < 8). The logits are recomputed from the partials with
// token_coeffs' arithmetic, so they are the forward's floats. Sinkhorn-Knopp
// is run forward again with each iterate M_k (before its column step) kept in
// LDS (`it_lds`, iters x 256 floats), then walked in reverse: for an iterate,
// A = T_c(M_k) and B = T_r(A) are recomputed from M_k and the gradient goes
// through T_r (g = (g - rowsum(g B)) / q) and then T_c (g = (g - colsum(g A)) /
// s); the logit gradient is g M_0 (the max subtracted before exp is a common
// factor, which Sinkhorn's output does not depend on). Gates: dz = dh s (1 - s)
// (pre) and 2 dh s (1 - s) (post) with s = sigmoid(z). Then with rho = 1/r:
// dP = alpha dz rho, d rho = sum alpha dz P, and the factor of vec x in its
// gradient, 2 dss = -d rho rho^3 / (4C) (0 for the all-zero state).
// Outputs per token: h_pre and h_res (the forward's maps, for the dX pass), dP
// [32] (columns 24..31 zero: the A operand of the dx product) and g2 (= 2 dss);
// per workgroup of 16 tokens, red [36] = the sums
// over its tokens of dz [32, zero past the map's columns] | dz P rho over the
// pre, post and res gates [3] | 0, which are then added over the workgroups for
// db and dalpha.
//
// LAY = 0: mHC, columns [pre 4 | post 4 | res 16], dh [T, 24].
// LAY = K (1 or 4): the xHC active set (k = 4) with K write-back components,
// columns [post 4K (a*K + j) | res 16] and dh [T, 4K + 16] in that order: lanes
// e < 4K carry post column e, no pre map (h_pre is not written).
//
// DHP (mHC): the partials come from proj_wide_kernel with DH (32 padded columns,
// then ss and the 4 sums <dF_in, x_i> per item): dH_pre = those sums added over
// the token's items in order, also stored into dh[:, 0:4].
template <int TT, int LAY, bool DHP = false>
__global__ __launch_bounds__(256) void bwd_coeff_kernel(const float* __restrict__ part, int64_t T, int64_t C, int S,
                                                        const float* __restrict__ bias, Gate gate, int iters,
                                                        float* __restrict__ dh, float* __restrict__ dP,
                                                        float* __restrict__ g2, float* __restrict__ red,
                                                        float* __restrict__ h_pre, float* __restrict__ h_res) {
  constexpr bool ROUTE = LAY != 0;
  constexpr int RES0 = ROUTE ? 4 * LAY : 8;  // first res column
  constexpr int NGC = RES0;                  // gate (pre/post) columns before it
  constexpr int DHS = RES0 + 16;             // dh row length
  static_assert(NGC == 4 || NGC == 8 || NGC == 16, "gate columns");
  static_assert(!DHP || !ROUTE, "the fused dH_pre sums are the mHC pre map's");
  extern __shared__ float it_lds[];  // [iters][256]
  using PG = PartGeom<(DHP || ROUTE ? 4 : 3), TT, DHP ? NS4 : 0>;
  const int tid = threadIdx.x;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + tid;
  const int64_t tt = g >> 4;
  const int e = (int)(g & 15);
  const bool valid = tt < T;
  const int64_t tc = valid ? tt : T - 1;
  const int64_t tile = tc / TT;
  const int m = (int)(tc - tile * TT);
  const float* base = part + tile * S * PG::PART + m * PG::PROW;
  float ss = 0.f, pr = 0.f, pe = 0.f, pd = 0.f;
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float* b = base + (int64_t)s * PG::PART;
    ss += b[PG::NCOLP];
    pr += b[RES0 + e];
    pe += b[e & (NGC - 1)];
    if constexpr (DHP) pd += b[PG::NCOLP + 1 + (e & 3)];
  }
  if constexpr (DHP) {
    if (valid && e < 4) dh[tt * DHS + e] = pd;
  }
  const float invr = inv_rms4(ss, C);
  const float a = (ROUTE || e >= 4) ? gate.a_post : gate.a_pre;
  const float sg = sigmoid(gate_logit(a, pe, invr, bias[e & (NGC - 1)]));
  const float z = gate_logit(gate.a_res, pr, invr, bias[RES0 + e]);
  float zm = fmaxf(z, dpp<DPP_QXOR1>(z));
  zm = fmaxf(zm, dpp<DPP_QXOR2>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR4>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR8>(zm));
  const float M0 = expf(z - zm);
  float M = M0;
  for (int it = 0; it < iters; ++it) {
    it_lds[it * 256 + tid] = M;
    float cs = M + dpp<DPP_ROR8>(M);
    cs += dpp<DPP_ROR4>(cs);
    M = M / cs;
    float rs = M + dpp<DPP_QXOR1>(M);
    rs += dpp<DPP_QXOR2>(rs);
    M = M / rs;
  }
  if (valid) {  // the forward's maps, for the dX pass
    h_res[tt * 16 + e] = M;
    if (!ROUTE && e < 4) h_pre[tt * 4 + e] = sg;
  }
  // each lane reads back only the iterates it wrote: no barrier needed
  float G = dh[tc * DHS + RES0 + e];
  for (int it = iters - 1; it >= 0; --it) {
    // (the reverse walk divides by one reciprocal per sum, v_rcp_f32 to 1 ulp)
    const float Mk = it_lds[it * 256 + tid];
    float cs = Mk + dpp<DPP_ROR8>(Mk);
    cs += dpp<DPP_ROR4>(cs);
    const float rcs = __builtin_amdgcn_rcpf(cs);
    const float A = Mk * rcs;
    float rs = A + dpp<DPP_QXOR1>(A);
    rs += dpp<DPP_QXOR2>(rs);
    const float rrs = __builtin_amdgcn_rcpf(rs);
    const float B = A * rrs;
    float u = G * B;  // through T_r: the row sum of G B
    u += dpp<DPP_QXOR1>(u);
    u += dpp<DPP_QXOR2>(u);
    G = (G - u) * rrs;
    float v = G * A;  // through T_c: the column sum of G A
    v += dpp<DPP_ROR8>(v);
    v += dpp<DPP_ROR4>(v);
    G = (G - v) * rcs;
  }
  const float dz_res = G * M0;
  float dz_pp = 0.f;
  if (e < NGC) {
    const float d = DHP && e < 4 ? pd : dh[tc * DHS + e];
    dz_pp = ((!ROUTE && e < 4) ? d : 2.0f * d) * sg * (1.0f - sg);
  }
  // sums over the 16 lanes: quads, then the four quads (every lane gets the total)
  auto row16 = [](float x) __attribute__((always_inline)) {
    x += dpp<DPP_QXOR1>(x);
    x += dpp<DPP_QXOR2>(x);
    x += dpp<DPP_ROR8>(x);
    x += dpp<DPP_ROR4>(x);
    return x;
  };
  const float drho = row16(gate.a_res * dz_res * pr + (e < NGC ? a * dz_pp * pe : 0.f));
  const float u_pre = ROUTE ? 0.f : row16(e < 4 ? dz_pp * pe * invr : 0.f);
  const float u_post = row16(e >= (ROUTE ? 0 : 4) && e < NGC ? dz_pp * pe * invr : 0.f);
  const float u_res = row16(dz_res * pr * invr);
  if (valid) {
    dP[tt * 32 + RES0 + e] = gate.a_res * dz_res * invr;
    if (e < NGC) dP[tt * 32 + e] = a * dz_pp * invr;
    if (e < 32 - RES0 - 16) dP[tt * 32 + RES0 + 16 + e] = 0.f;
    if (e == 0) g2[tt] = -drho * invr * invr * invr / (float)(NS4 * C);
  }
  // the workgroup's 16 tokens added in token order (rows past T add zero)
  __shared__ float bsum[16][36];
  const int tk = tid >> 4;
  bsum[tk][RES0 + e] = valid ? dz_res : 0.f;
  if (e < NGC) bsum[tk][e] = valid ? dz_pp : 0.f;
  if (e < 16 - RES0) bsum[tk][RES0 + 16 + e] = 0.f;
  if (e < 4) bsum[tk][32 + e] = !valid || e == 3 ? 0.f : (e == 0 ? u_pre : (e == 1 ? u_post : u_res));
  __syncthreads();
  if (tid < 36) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) sum += bsum[k][tid];
    red[(int64_t)blockIdx.x * 36 + tid] = sum;
  }
}

// Backward of the xHC pre map h_pre = sigmoid(alpha_pre P / r + b_pre) for token
// tt, from the full-state partials of proj_wide_kernel with DH (per tile the N/4
// stream groups x S slices, columns [pre N | ... | ss | <dF_in, x_i> of the
// group's 4 streams]). 16 lanes per token, lane c < N for pre column c: P and
// the sum of squares added over the items in order, dH_pre[c] = <dF_in, x_c>
// added over the S items of c's group in order, r = sqrt(ss / (N C)) and h_pre
// as xpre_finish_kernel forms them, then dz = dH_pre h (1 - h), dP = alpha dz /
// r and the gradient through r, 2 dss = -d rho rho^3 / (N C). Outputs: dh_pre
// [T, N], dP [T, 32] (columns N..31 zero), g2, h_pre [T, N], and per workgroup
// of 16 tokens red [36] = the sums of dz [16, zero past N] | 0 x 16 | dz P rho
// over the gate | 0 0 0.
template <int NB, int TT>
__global__ __launch_bounds__(256) void bwd_xpre_coeff_kernel(const float* __restrict__ part, int64_t T, int64_t C,
                                                             int N, int S, const float* __restrict__ b_pre,
                                                             float a_pre, float* __restrict__ dh_pre,
                                                             float* __restrict__ dP, float* __restrict__ g2,
                                                             float* __restrict__ red, float* __restrict__ h_pre) {
  using PG = PartGeom<NB, TT, NS4>;
  const int per_tile = (N / 4) * S;
  const int tid = threadIdx.x;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + tid;
  const int64_t tt = g >> 4;
  const int c = (int)(g & 15);
  const bool valid = tt < T;
  const int64_t tc = valid ? tt : T - 1;
  const int64_t tile = tc / TT;
  const int mrow = (int)(tc - tile * TT);
  const float* base = part + tile * per_tile * PG::PART + mrow * PG::PROW;
  const int cc = c < N ? c : 0;
  float ss = 0.f, pc = 0.f, dhc = 0.f;
#pragma unroll 4
  for (int it = 0; it < per_tile; ++it) {
    const float* b = base + (int64_t)it * PG::PART;
    ss += b[PG::NCOLP];
    pc += b[cc];
  }
  {
    const float* b = base + (int64_t)(cc >> 2) * S * PG::PART + PG::NCOLP + 1 + (cc & 3);
#pragma unroll 4
    for (int it = 0; it < S; ++it) dhc += b[(int64_t)it * PG::PART];
  }
  const float r = sqrtf(ss / (float)((double)N * (double)C));
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  const bool col = c < N;
  const float h = sigmoid(a_pre * (pc * invr) + b_pre[cc]);
  const float dz = col ? dhc * h * (1.0f - h) : 0.f;
  const float drho = row16_sum(a_pre * dz * pc);
  const float u = row16_sum(dz * pc * invr);
  if (valid) {
    if (col) dh_pre[tt * N + c] = dhc;
    dP[tt * 32 + c] = col ? a_pre * dz * invr : 0.f;
    dP[tt * 32 + 16 + c] = 0.f;
    if (col) h_pre[tt * N + c] = h;
    if (c == 0) g2[tt] = -drho * invr * invr * invr / (float)((double)N * (double)C);
  }
  __shared__ float bsum[16][36];
  const int tk = tid >> 4;
  bsum[tk][c] = valid ? dz : 0.f;
  bsum[tk][16 + c] = 0.f;
  if (c < 4) bsum[tk][32 + c] = (c == 0 && valid) ? u : 0.f;
  __syncthreads();
  if (tid < 36) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) sum += bsum[k][tid];
    red[(int64_t)blockIdx.x * 36 + tid] = sum;
  }
}

// ------------------------------------------------------- xHC finish kernels

// xHC full-state pass ([xHC] steps 1 and 2, parameterisation): 32 lanes per
// token, lane c owns column c of the projection [pre npre | router nr]. Each
// lane adds the token's items in order (column c and the sum of squares), then
// r = sqrt(ss / (N C)); pre lanes: h_pre = sigmoid(alpha_pre P / r + b_pre);
// router lanes: score = sigmoid(P / r). Selection (when nr > 0): k - m rounds
// of an arg-max over the candidate lanes (equal scores go to the lower stream),
// then idx = the m fixed streams and the chosen ones in ascending order.
// With PAIRP the projection is split in two: the partials `part` cover the
// rows left out of the previous route's active set (the carry of the chained
// step), and the pair partials pp (PAIRS items, ps slices per pair tile) the
// active rows, pair pos[t, j] for slot j (< 0: none); both are added per token.
template <int NB, int TT, bool PAIRP = false>
__global__ __launch_bounds__(256) void xpre_finish_kernel(const float* __restrict__ part, int64_t T, int64_t C, int N,
                                                          int per_tile, int npre, int nr, int k, int m,
                                                          const float* __restrict__ b_pre, float a_pre,
                                                          float* __restrict__ h_pre, float* __restrict__ score,
                                                          int32_t* __restrict__ idx, const float* __restrict__ pp = nullptr,
                                                          const int32_t* __restrict__ ppos = nullptr, int pk = 0,
                                                          int ps = 0) {
  using PG = PartGeom<NB, TT>;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tt = g >> 5;
  const int c = (int)(g & 31);
  const int64_t tc = tt < T ? tt : T - 1;
  const int64_t tile = tc / TT;
  const int mrow = (int)(tc - tile * TT);
  const float* base = part + tile * per_tile * PG::PART + mrow * PG::PROW;
  const int cc = c < PG::NCOLP ? c : 0;
  float ss = 0.f, pc = 0.f;
#pragma unroll 4
  for (int it = 0; it < per_tile; ++it) {
    const float* b = base + (int64_t)it * PG::PART;
    ss += b[PG::NCOLP];
    pc += b[cc];
  }
  if constexpr (PAIRP) {
    for (int j = 0; j < pk; ++j) {
      const int pq = ppos[tc * pk + j];
      if (pq < 0) continue;
      const float* b = pp + (int64_t)(pq / TT) * ps * PG::PART + (pq % TT) * PG::PROW;
      for (int sl = 0; sl < ps; ++sl) {
        ss += b[(int64_t)sl * PG::PART + PG::NCOLP];
        pc += b[(int64_t)sl * PG::PART + cc];
      }
    }
  }
  const float r = sqrtf(ss / (float)((double)N * (double)C));
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  const bool valid = tt < T;
  const bool is_pre = c < npre, is_rt = c >= npre && c < npre + nr;
  if (valid && is_pre && h_pre) h_pre[tt * npre + c] = sigmoid(a_pre * (pc * invr) + b_pre[c]);
  if (nr == 0) return;  // uniform over the launch
  const float sc = sigmoid(pc * invr);
  if (valid && is_rt) score[tt * nr + (c - npre)] = sc;
  // arg-max rounds within the 32-lane group: (key, candidate) ordered by key,
  // then by the lower candidate; the butterfly leaves the winner in every lane
  float key = is_rt ? sc : -1.f;
  const int cand = is_rt ? c - npre : 64;
  uint64_t chosen = 0;
  for (int round = 0; round < k - m; ++round) {
    float bv = key;
    int bl = cand;
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 32);
      const int ol = __shfl_xor(bl, d, 32);
      if (ov > bv || (ov == bv && ol < bl)) {
        bv = ov;
        bl = ol;
      }
    }
    chosen |= 1ull << (m + bl);  // candidate j is stream m + j
    if (cand == bl) key = -2.f;
  }
  if (valid && c < k) {
    const uint64_t mask = chosen | ((m >= 64 ? ~0ull : (1ull << m) - 1));
    int cnt = 0, v = 0;
    for (int sidx = 0; sidx < N; ++sidx)
      if ((mask >> sidx) & 1ull) {
        if (cnt == c) v = sidx;
        ++cnt;
      }
    idx[tt * k + c] = v;
  }
}

// xHC-Flash block entry ([xHC] xHC-Flash variant: the router once and every
// sublayer's pre map from the block-entry state): the finish of the one
// projection pass over columns [router N - m | pre map 0, N | ... | pre map L-1].
// 32 lanes per token; lane c takes columns c, c + 32, c + 64 (each summed over
// the token's items in order, as xpre_finish_kernel does), the router lanes c <
// N - m run the same arg-max rounds.
template <int NB>
__global__ __launch_bounds__(256) void flash_entry_finish_kernel(const float* __restrict__ part, int64_t T,
                                                                 int64_t C, int N, int per_tile, int L, int k, int m,
                                                                 const float* __restrict__ b_pre, float a_pre,
                                                                 float* __restrict__ h_pre, float* __restrict__ score,
                                                                 int32_t* __restrict__ idx) {
  using PG = PartGeom<NB, W_TOK>;
  constexpr int NJ = (PG::NCOLP + 31) / 32;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tt = g >> 5;
  const int c = (int)(g & 31);
  const int64_t tc = tt < T ? tt : T - 1;
  const int64_t tile = tc / W_TOK;
  const int mrow = (int)(tc - tile * W_TOK);
  const float* base = part + tile * per_tile * PG::PART + mrow * PG::PROW;
  float ss = 0.f, pc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) pc[j] = 0.f;
#pragma unroll 2
  for (int it = 0; it < per_tile; ++it) {
    const float* b = base + (int64_t)it * PG::PART;
    ss += b[PG::NCOLP];
#pragma unroll
    for (int j = 0; j < NJ; ++j) pc[j] += b[c + 32 * j < PG::NCOLP ? c + 32 * j : 0];
  }
  const float r = sqrtf(ss / (float)((double)N * (double)C));
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  const bool valid = tt < T;
  const int nr = N - m;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int col = c + 32 * j - nr;
    if (valid && col >= 0 && col < L * N) {
      const int l = col / N, i = col - l * N;
      h_pre[((int64_t)l * T + tt) * N + i] = sigmoid(a_pre * (pc[j] * invr) + b_pre[l * N + i]);
    }
  }
  const bool is_rt = c < nr;
  const float sc = sigmoid(pc[0] * invr);
  if (valid && is_rt && score) score[tt * nr + c] = sc;
  float key = is_rt ? sc : -1.f;
  const int cand = is_rt ? c : 64;
  uint64_t chosen = 0;
  for (int round = 0; round < k - m; ++round) {
    float bv = key;
    int bl = cand;
#pragma unroll
    for (int d = 16; d >= 1; d >>= 1) {
      const float ov = __shfl_xor(bv, d, 32);
      const int ol = __shfl_xor(bl, d, 32);
      if (ov > bv || (ov == bv && ol < bl)) {
        bv = ov;
        bl = ol;
      }
    }
    chosen |= 1ull << (m + bl);
    if (cand == bl) key = -2.f;
  }
  if (valid && c < k) {
    const uint64_t mask = chosen | ((m >= 64 ? ~0ull : (1ull << m) - 1));
    int cnt = 0, v = 0;
    for (int sidx = 0; sidx < N; ++sidx)
      if ((mask >> sidx) & 1ull) {
        if (cnt == c) v = sidx;
        ++cnt;
      }
    idx[tt * k + c] = v;
  }
}

// xHC active coefficients ([xHC] step 3, parameterisation) for k = 4: 16 lanes
// per token. Columns [post k*K (a*K + j) | res 16 (a*4 + b)]. Each lane adds the
// token's items in order, r_A = sqrt(ss / (4 C)); post lanes e < 4K: H_post =
// 2 sigmoid(alpha_post P / r + b); H_res = Sinkhorn-Knopp(exp(alpha_res P / r +
// b)) on the 4x4 block held by the 16 lanes (DPP exchanges as in mHC).
// TT: tokens per item of the partials.
template <int NB, int TT = TILE>
__global__ __launch_bounds__(256) void xroute_finish_kernel(const float* __restrict__ part, int64_t T, int64_t C,
                                                            int per_tile, int K, const float* __restrict__ b_act,
                                                            float a_post, float a_res, int iters,
                                                            float* __restrict__ Hp, float* __restrict__ Hr) {
  using PG = PartGeom<NB, TT>;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tt = g >> 4;
  const int e = (int)(g & 15);
  const int64_t tc = tt < T ? tt : T - 1;
  const int64_t tile = tc / TT;
  const int mrow = (int)(tc - tile * TT);
  const float* base = part + tile * per_tile * PG::PART + mrow * PG::PROW;
  const int kK = 4 * K;  // post entries: lane e takes e and, for K > 4, e + 16
  const int cpost = e < kK ? e : 0, cpost2 = e + 16 < kK ? e + 16 : 0;
  float ss = 0.f, pr = 0.f, pp = 0.f, pp2 = 0.f;
#pragma unroll 4
  for (int it = 0; it < per_tile; ++it) {
    const float* b = base + (int64_t)it * PG::PART;
    ss += b[PG::NCOLP];
    pr += b[kK + e];
    pp += b[cpost];
    if (PG::NCOLP > 32) pp2 += b[cpost2];
  }
  const float r = sqrtf(ss / (float)(4.0 * (double)C));
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  const bool valid = tt < T;
  if (valid && e < kK) Hp[tt * kK + e] = 2.0f * sigmoid(a_post * (pp * invr) + b_act[e]);
  if (valid && e + 16 < kK) Hp[tt * kK + e + 16] = 2.0f * sigmoid(a_post * (pp2 * invr) + b_act[e + 16]);
  const float z = a_res * (pr * invr) + b_act[kK + e];
  float zm = fmaxf(z, dpp<DPP_QXOR1>(z));
  zm = fmaxf(zm, dpp<DPP_QXOR2>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR4>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR8>(zm));
  float M = expf(z - zm);
  for (int it = 0; it < iters; ++it) {
    float cs = M + dpp<DPP_ROR8>(M);  // column sum over a
    cs += dpp<DPP_ROR4>(cs);
    M = M / cs;
    float rs = M + dpp<DPP_QXOR1>(M);  // row sum over b
    rs += dpp<DPP_QXOR2>(rs);
    M = M / rs;
  }
  if (valid) Hr[tt * 16 + e] = M;
}

// --------------------------------------------------------------- pre-read

// F_in[t, c] = sum_i h_pre[t, i] X[t, i, c] for n = 4 bf16; 8 channels per thread.
__global__ __launch_bounds__(256) void pre4_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t C,
                                                   const float* __restrict__ h_pre,
                                                   uint16_t* __restrict__ F_in) {
  const int64_t nch = C / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const float w0 = h_pre[t * 4 + 0], w1 = h_pre[t * 4 + 1], w2 = h_pre[t * 4 + 2], w3 = h_pre[t * 4 + 3];
  const uint16_t* p = X + t * 4 * C + c0;
  float a[8], b[8], c[8], d[8], o[8];
  unpack8(ld_stream(p), a);
  unpack8(ld_stream(p + C), b);
  unpack8(ld_stream(p + 2 * C), c);
  unpack8(ld_stream(p + 3 * C), d);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = w0 * a[e] + w1 * b[e] + w2 * c[e] + w3 * d[e];
  // F_in is not read again by this pass: a nontemporal store
  __builtin_nontemporal_store(u32x4_t{pack_bf2_hw(o[0], o[1]), pack_bf2_hw(o[2], o[3]), pack_bf2_hw(o[4], o[5]),
                                      pack_bf2_hw(o[6], o[7])},
                              reinterpret_cast<u32x4_t*>(F_in + t * C + c0));
}

// h_pre of token tt ([mHC] Eq. 15-18) from the partial projections, with the
// arithmetic of token_coeffs (slices added in order, the same gate helpers), so
// both give the same floats.
template <int TT>
__device__ __forceinline__ void token_pre4(const float* __restrict__ part, int64_t tt, int64_t C, int S,
                                           const float* __restrict__ bias, float a_pre, float (&w)[4]) {
  using PG = PartGeom<3, TT>;
  const int64_t tile = tt / TT;
  const int m = (int)(tt - tile * TT);
  const float* base = part + tile * S * PG::PART + m * PG::PROW;
  float ss = 0.f, pe[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = 0; s < S; ++s) {
    const float* b = base + (int64_t)s * PG::PART;
    ss += b[PG::NCOLP];
#pragma unroll
    for (int e = 0; e < 4; ++e) pe[e] += b[e];
  }
  const float invr = inv_rms4(ss, C);
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = sigmoid(gate_logit(a_pre, pe[e], invr, bias[e]));
}

// The finish and the pre-read in one launch. Blocks [0, ncb) are
// coeffs_finish_kernel (16 threads per token); the others are pre4_kernel,
// each thread forming its token's h_pre from the partials itself instead of
// waiting for the finish blocks. The two kinds of block are independent, so
// the latency-bound finish runs beside the bandwidth-bound pre-read. The
// pre-read blocks take the tokens from the last to the first: the split pass
// before wrote the state tile by tile from the first, so the rows it wrote
// last (the likeliest to be still in the last-level cache) are read first,
// and the pass ends on the first rows, where the next split pass begins.
template <int TT>
__global__ __launch_bounds__(256) void finish_pre4_kernel(const float* __restrict__ part, int64_t T, int64_t C, int S,
                                                          const float* __restrict__ bias, Gate gate, int iters,
                                                          float* __restrict__ h_pre_out,
                                                          float* __restrict__ h_post_out,
                                                          float* __restrict__ h_res_out, int ncb,
                                                          const uint16_t* __restrict__ X,
                                                          uint16_t* __restrict__ F_in) {
  if ((int)blockIdx.x < ncb) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t tt = g >> 4;
    token_coeffs<TT>(part, tt < T ? tt : T - 1, (int)(g & 15), C, S, bias, gate, iters, tt < T, h_pre_out,
                     h_post_out, h_res_out);
    return;
  }
  const int64_t nch = C / 8;
  const int64_t g = (int64_t)((int)gridDim.x - 1 - (int)blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= T * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const uint16_t* p = X + t * 4 * C + c0;
  const uint4 x0 = ld_stream(p), x1 = ld_stream(p + C), x2 = ld_stream(p + 2 * C), x3 = ld_stream(p + 3 * C);
  float w[4];
  token_pre4<TT>(part, t, C, S, bias, gate.a_pre, w);
  float a[8], b[8], c[8], d[8], o[8];
  unpack8(x0, a);
  unpack8(x1, b);
  unpack8(x2, c);
  unpack8(x3, d);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = w[0] * a[e] + w[1] * b[e] + w[2] * c[e] + w[3] * d[e];
  __builtin_nontemporal_store(u32x4_t{pack_bf2_hw(o[0], o[1]), pack_bf2_hw(o[2], o[3]), pack_bf2_hw(o[4], o[5]),
                                      pack_bf2_hw(o[6], o[7])},
                              reinterpret_cast<u32x4_t*>(F_in + t * C + c0));
}

// F_in[t, c] = sum_i h_pre[t, i] X[t, i, c] over NS bfloat16 streams (the xHC
// full-state pre-read, [xHC] step 2); 8 channels per thread, all NS rows in
// flight at once. Blocks take the tokens from the last to the first, so the
// rows the projection pass read last are read first.
template <int NS, bool H16>  // H16: h_pre is 16-byte aligned (read as float4)
__global__ __launch_bounds__(256) void pre_wide_kernel(const uint16_t* __restrict__ X, int64_t T, int64_t C,
                                                       const float* __restrict__ h_pre,
                                                       uint16_t* __restrict__ F_in) {
  const int64_t nch = C / 8;
  const int64_t g = (int64_t)((int)gridDim.x - 1 - (int)blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= T * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const uint16_t* p = X + t * NS * C + c0;
  uint4 x[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) x[i] = ld_stream(p + i * C);
  float w[NS];
  if (H16) {
    const float4* hp = reinterpret_cast<const float4*>(h_pre + t * NS);
#pragma unroll
    for (int i = 0; i < NS / 4; ++i) {
      const float4 v = hp[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NS; ++i) w[i] = h_pre[t * NS + i];
  }
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    float xv[8];
    unpack8(x[i], xv);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] += w[i] * xv[e];
  }
  __builtin_nontemporal_store(u32x4_t{pack_bf2_hw(o[0], o[1]), pack_bf2_hw(o[2], o[3]), pack_bf2_hw(o[4], o[5]),
                                      pack_bf2_hw(o[6], o[7])},
                              reinterpret_cast<u32x4_t*>(F_in + t * C + c0));
}

// xHC mix + scatter for k = 4 bfloat16 active streams and K <= 8 write-back
// components, in place ([xHC] step 3): X[t, idx[a]] = sum_b H_res[t, a, b]
// X[t, idx[b]] + sum_j H_post[t, a, j] Wb[t, j], 8 channels per thread, all
// 4 + K rows in flight at once, nontemporal loads and stores (each row is read
// and written once here). Tokens with an index outside [0, N) are left
// unchanged. Blocks take the tokens from the last to the first: the projection
// pass before read the gathered rows from the first token on, so the rows it
// read last are read first here.
//
// Components j >= j0 may come from a second array Wb2 [T, K - j0, C] (an
// xHC-Flash block whose last sublayer's components are kept apart); rows j <
// j0 are read from Wb [T, K, C].
template <int K, bool SPLIT = false>
__global__ __launch_bounds__(256) void mix4_kernel(uint16_t* X, int64_t T, int N, int64_t C,
                                                   const int32_t* __restrict__ idx,
                                                   const float* __restrict__ H_res,
                                                   const float* __restrict__ H_post,
                                                   const uint16_t* __restrict__ Wb,
                                                   const uint16_t* __restrict__ Wb2, int j0) {
  const int64_t nch = C / 8;
  const int64_t g = (int64_t)((int)gridDim.x - 1 - (int)blockIdx.x) * blockDim.x + threadIdx.x;
  if (g >= T * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  int s[4];
  bool ok = true;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    s[a] = idx[t * 4 + a];
    ok = ok && s[a] >= 0 && s[a] < N;
  }
  if (!ok) return;
  uint4 xr[4], wr[K];
#pragma unroll
  for (int a = 0; a < 4; ++a) xr[a] = ld_stream(X + (t * N + s[a]) * C + c0);
#pragma unroll
  for (int j = 0; j < K; ++j)
    wr[j] = ld_stream(!SPLIT || j < j0 ? Wb + (t * K + j) * C + c0 : Wb2 + (t * (K - j0) + (j - j0)) * C + c0);
  const float* hr = H_res + t * 16;
  const float* hp = H_post + t * 4 * K;
  float x[4][8], y[4][8];
#pragma unroll
  for (int b = 0; b < 4; ++b) unpack8(xr[b], x[b]);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[a][e] = 0.f;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float w = hr[a * 4 + b];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[a][e] += w * x[b][e];
    }
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    float wv[8];
    unpack8(wr[j], wv);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float w = hp[a * K + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[a][e] += w * wv[e];
    }
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    uint4 o;
    o.x = pack_bf2_hw(y[a][0], y[a][1]);
    o.y = pack_bf2_hw(y[a][2], y[a][3]);
    o.z = pack_bf2_hw(y[a][4], y[a][5]);
    o.w = pack_bf2_hw(y[a][6], y[a][7]);
    __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w},
                                reinterpret_cast<u32x4_t*>(X + (t * N + s[a]) * C + c0));
  }
}

// ------------------------------------------------------ active-row pairs

// The pairs (t, j) of an active set idx [T, k] grouped by stream: bucket z holds
// the pairs whose row is stream z, padded to whole tiles of W_TOK pairs. Three
// launches over blocks of SORT_THR tokens: (1) each block's pairs per stream (a
// wave counts its lanes with one ballot per stream, the waves' counts added in
// order); (2) the buckets' first tiles (tile_off [N + 1], tile_off[N] the tiles
// used), each block's first slot per stream, and the padding: ptok = -1 for the
// tail of each bucket's last tile and every slot past the last bucket up to
// ntile tiles; (3) each block places its pairs, slot order (block, slot j,
// wave, lane): ptok (the token of each slot) and pos [T, k] (each pair's slot;
// -1 for an index outside [0, N)).
constexpr int SORT_THR = 256;
constexpr int SORT_NW = SORT_THR / 64;
constexpr int SORT_MAXN = 16;

__global__ __launch_bounds__(SORT_THR) void pair_count_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int N,
                                                              int32_t* __restrict__ cnt) {
  __shared__ int wc[SORT_NW][SORT_MAXN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = (int64_t)blockIdx.x * SORT_THR + tid;
  int mine = 0;  // lane y: the wave's pairs of stream y
  for (int j = 0; j < k; ++j) {
    const int z = t < T ? idx[t * k + j] : -1;
    for (int y = 0; y < N; ++y) {
      const uint64_t mk = __ballot(z == y);
      if (lane == y) mine += __popcll(mk);
    }
  }
  if (lane < N) wc[wave][lane] = mine;
  __syncthreads();
  if (tid < N) {
    int sum = 0;
    for (int w = 0; w < SORT_NW; ++w) sum += wc[w][tid];
    cnt[(int64_t)blockIdx.x * N + tid] = sum;
  }
}

// (G * N counts, staged through LDS in chunks so the per-stream sums run on LDS)
constexpr int SCAN_CHUNK = 4096;
__global__ __launch_bounds__(SORT_THR) void pair_scan_kernel(const int32_t* __restrict__ cnt, int G, int N, int ntile,
                                                             int32_t* __restrict__ tile_off,
                                                             int32_t* __restrict__ base,
                                                             int32_t* __restrict__ ptok) {
  __shared__ int total[SORT_MAXN], first[SORT_MAXN + 1];
  __shared__ int stage[SCAN_CHUNK];
  const int tid = threadIdx.x;
  const int64_t nc = (int64_t)G * N;
  const int bpc = SCAN_CHUNK / N;  // blocks per chunk
  int run = 0;
  for (int64_t c0 = 0; c0 < nc; c0 += (int64_t)bpc * N) {
    const int64_t n = nc - c0 < (int64_t)bpc * N ? nc - c0 : (int64_t)bpc * N;
    __syncthreads();
    for (int i = tid; i < n; i += SORT_THR) stage[i] = cnt[c0 + i];
    __syncthreads();
    if (tid < N)
      for (int b = 0; b < n / N; ++b) run += stage[b * N + tid];
  }
  if (tid < N) total[tid] = run;
  __syncthreads();
  if (tid == 0) {
    int f = 0;
    for (int z = 0; z < N; ++z) {
      first[z] = f;
      f += (total[z] + W_TOK - 1) / W_TOK;
    }
    first[N] = f;
  }
  __syncthreads();
  if (tid <= N) tile_off[tid] = first[tid];
  run = tid < N ? first[tid] * W_TOK : 0;
  for (int64_t c0 = 0; c0 < nc; c0 += (int64_t)bpc * N) {
    const int64_t n = nc - c0 < (int64_t)bpc * N ? nc - c0 : (int64_t)bpc * N;
    __syncthreads();
    for (int i = tid; i < n; i += SORT_THR) stage[i] = cnt[c0 + i];
    __syncthreads();
    if (tid < N)
      for (int b = 0; b < n / N; ++b) {
        const int v = stage[b * N + tid];
        stage[b * N + tid] = run;
        run += v;
      }
    __syncthreads();
    for (int i = tid; i < n; i += SORT_THR) base[c0 + i] = stage[i];
  }
  for (int z = 0; z < N; ++z) {
    const int a = first[z] * W_TOK + total[z], e = first[z + 1] * W_TOK;
    for (int i = a + tid; i < e; i += SORT_THR) ptok[i] = -1;
  }
  for (int64_t i = (int64_t)first[N] * W_TOK + tid; i < (int64_t)ntile * W_TOK; i += SORT_THR) ptok[i] = -1;
}

__global__ __launch_bounds__(SORT_THR) void pair_place_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int N,
                                                              const int32_t* __restrict__ base,
                                                              int32_t* __restrict__ ptok, int32_t* __restrict__ pos) {
  __shared__ int wc[SORT_NW][SORT_MAXN], woff[SORT_NW][SORT_MAXN], run[SORT_MAXN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int64_t t = (int64_t)blockIdx.x * SORT_THR + tid;
  if (tid < N) run[tid] = base[(int64_t)blockIdx.x * N + tid];
  for (int j = 0; j < k; ++j) {
    const int z0 = t < T ? idx[t * k + j] : -1;
    const int z = z0 >= 0 && z0 < N ? z0 : -1;
    int rank = 0;
    for (int y = 0; y < N; ++y) {
      const uint64_t mk = __ballot(z == y);
      if (z == y) rank = __popcll(mk & below);
      if (lane == y) wc[wave][y] = __popcll(mk);
    }
    __syncthreads();  // (also orders the first slot after run's initialisation)
    if (tid < N) {
      int r = run[tid];
      for (int w = 0; w < SORT_NW; ++w) {
        woff[w][tid] = r;
        r += wc[w][tid];
      }
      run[tid] = r;
    }
    __syncthreads();
    if (t < T) {
      int slot = -1;
      if (z >= 0) {
        slot = woff[wave][z] + rank;
        ptok[slot] = (int32_t)t;
      }
      pos[t * k + j] = slot;
    }
    __syncthreads();  // wc and woff are rewritten for the next slot
  }
}

// ----------------------------------------------------------------- hosts

static inline bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

namespace {
struct Geom {
  int NG, S, nitem;  // stream groups, channel slices per group, items
};
// Both item kinds cover SPI * SC = W_SPI * W_SC = 1024 channels of a stream
// group, so a token's slices are the same for either; TT is the item's tokens.
static_assert(SPI * SC == W_SPI * W_SC, "channels per item");
int64_t slices(int64_t C) { return (C + SPI * SC - 1) / (SPI * SC); }
Geom geom(int64_t T, int64_t C, int NG, int TT) {
  const int64_t S = slices(C);
  return Geom{NG, (int)S, (int)(((T + TT - 1) / TT) * NG * S)};
}
// Tokens rounded up to whole W_TOK-token items: the partial buffer sized for
// them holds the partials of either item size.
int64_t part_tokens(int64_t T) { return (T + W_TOK - 1) / W_TOK * W_TOK; }
// the shapes the split kernels address with 32-bit buffer offsets and int item ids
bool shape_ok(int64_t T, int64_t C, int NG, int NB) {
  if (C % 32 != 0 || C < 32 || C >= (1ll << 24)) return false;
  return part_tokens(T) * NG * slices(C) * (NB * 8 + 1) * 4 < (1ll << 31);
}
int64_t part_bytes(int64_t T, int64_t C, int NG, int NB, int EX = 0) {
  return part_tokens(T) * NG * slices(C) * (NB * 8 + 1 + EX) * 4;
}
int nb_for(int ncols) { return ncols <= 16 ? 2 : (ncols <= 24 ? 3 : 4); }
int grid_for(int nitem) {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    ncu = 256;
  return nitem < ncu ? nitem : ncu;
}
// The same number of item rounds with every workgroup taking one item per round
// (528 items on 256 CUs: 176 workgroups of 3 items, not 16 of the 256 taking a
// third round alone).
int grid_balanced(int nitem) {
  const int g = grid_for(nitem);
  const int rounds = (nitem + g - 1) / g;
  return (nitem + rounds - 1) / rounds;
}

SplitArgs args(const void* X, int64_t T, int64_t C, int64_t rowstride, const Geom& g, const void* phi_p,
               float* part) {
  SplitArgs A{};
  A.X = (const uint16_t*)X;
  A.T = T;
  A.C = C;
  A.rowstride = rowstride;
  A.NG = g.NG;
  A.S = g.S;
  A.nitem = g.nitem;
  A.phi_p = (const uint16_t*)phi_p;
  A.part = part;
  return A;
}

template <bool POST, int NB, int MODE>
hipError_t launch_split(const SplitArgs& A, hipStream_t st) {
  hipLaunchKernelGGL((mhc_split_kernel<POST, NB, MODE>), dim3(grid_for(A.nitem)), dim3(STHR), 0, st, A);
  return hipGetLastError();
}

// the gathered active set beyond 32 columns (K > 4): NB = 5 or 6 blocks
hipError_t launch_split_gather(int nb, const SplitArgs& A, hipStream_t st) {
  return nb == 5 ? launch_split<false, 5, ROWS_GATHER>(A, st) : launch_split<false, 6, ROWS_GATHER>(A, st);
}

// projection only, W_TOK-token items (A from geom(..., W_TOK)); DH: with the
// dF_in sums (A.dF)
template <int NB, int MODE, bool DH = false>
hipError_t launch_wide(const SplitArgs& A, hipStream_t st) {
  hipLaunchKernelGGL((proj_wide_kernel<NB, MODE, DH>), dim3(grid_for(A.nitem)), dim3(STHR), 0, st, A);
  return hipGetLastError();
}

hipError_t launch_pack(const float* phi_a, int na, const float* phi_b, int nb, int64_t K, int ncolp, void* packed,
                       hipStream_t st, uint4* rows_out = nullptr) {
  hipLaunchKernelGGL(pack_phi_kernel, dim3((unsigned)(K / 64)), dim3(256), 0, st, phi_a, na, phi_b, nb, ncolp,
                     (uint16_t*)packed, rows_out);
  return hipGetLastError();
}

template <int TT>
hipError_t launch_finish(const float* part, int64_t T, int64_t C, int S, const float* bias, Gate gate, int iters,
                         float* h_pre, float* h_post, float* h_res, hipStream_t st) {
  const int64_t threads = T * 16;
  hipLaunchKernelGGL(coeffs_finish_kernel<TT>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, part, T, C, S,
                     bias, gate, iters, h_pre, h_post, h_res);
  return hipGetLastError();
}

template <int TT>
hipError_t launch_finish_pre4(const float* part, int64_t T, int64_t C, int S, const float* bias, Gate gate,
                              int iters, float* h_pre, float* h_post, float* h_res, const void* X, void* F_in,
                              hipStream_t st) {
  const int64_t ncb = (T * 16 + 255) / 256, npb = (T * (C / 8) + 255) / 256;
  hipLaunchKernelGGL(finish_pre4_kernel<TT>, dim3((unsigned)(ncb + npb)), dim3(256), 0, st, part, T, C, S, bias, gate,
                     iters, h_pre, h_post, h_res, (int)ncb, (const uint16_t*)X, (uint16_t*)F_in);
  return hipGetLastError();
}

// N % 4 == 0, 4 <= N <= 16, C % 8 == 0, X, F_in 16-byte aligned, h_pre [T, N]
hipError_t launch_pre_wide(const void* X, int64_t T, int N, int64_t C, const float* h_pre, void* F_in,
                           hipStream_t st) {
  const dim3 grid((unsigned)((T * (C / 8) + 255) / 256)), blk(256);
  const uint16_t* x = (const uint16_t*)X;
  uint16_t* f = (uint16_t*)F_in;
  const bool h16 = a16(h_pre);
#define HC_PRE_WIDE(NS)                                                                                     \
  if (h16) hipLaunchKernelGGL((pre_wide_kernel<NS, true>), grid, blk, 0, st, x, T, C, h_pre, f);          \
  else hipLaunchKernelGGL((pre_wide_kernel<NS, false>), grid, blk, 0, st, x, T, C, h_pre, f);
  switch (N) {
    case 4: HC_PRE_WIDE(4) break;
    case 8: HC_PRE_WIDE(8) break;
    case 12: HC_PRE_WIDE(12) break;
    default: HC_PRE_WIDE(16) break;
  }
#undef HC_PRE_WIDE
  return hipGetLastError();
}

hipError_t launch_pre4(const void* X, int64_t T, int64_t C, const float* h_pre, void* F_in, hipStream_t st) {
  const int64_t work = T * (C / 8);
  hipLaunchKernelGGL(pre4_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st, (const uint16_t*)X, T,
                     C, h_pre, (uint16_t*)F_in);
  return hipGetLastError();
}
}  // namespace

// ------------------------------------------------------------------ mHC

int64_t fast_coeffs_packed_bytes(int n, int64_t C, int dtype) {
  if (n != 4 || dtype != 1 || C % 32 != 0) return 0;
  return (int64_t)n * C / 8 * 48 * 16;
}

int64_t fast_coeffs_partial_bytes(int64_t T, int n, int64_t C, int dtype) {
  if (n != 4 || dtype != 1 || !shape_ok(T, C, 1, 3)) return 0;
  return part_bytes(T, C, 1, 3);
}

bool fast_coeffs_supported(int dtype, int n, int64_t T, int64_t C, const void* X) {
  return dtype == 1 && n == 4 && shape_ok(T, C, 1, 3) && a16(X);
}

bool fast_post_supported(int dtype, int n, int64_t C, const void* X, const void* F, const void* Y) {
  return dtype == 1 && n == 4 && C % 32 == 0 && C >= 32 && a16(X) && a16(F) && a16(Y);
}

hipError_t launch_fast_coeffs_pre(const void* X, int64_t T, int64_t C, const float* phi,
                                  const float* bias, float a_pre, float a_post, float a_res,
                                  int iters, float* h_pre, float* h_post, float* h_res, void* F_in,
                                  void* packed, float* partial, hipStream_t st) {
  hipError_t e = launch_pack(phi, NCOL, nullptr, 0, 4 * C, 24, packed, st);
  if (e != hipSuccess) return e;
  const Geom g = geom(T, C, 1, W_TOK);
  if ((e = launch_wide<3, ROWS_CONTIG>(args(X, T, C, 4 * C, g, packed, partial), st)) != hipSuccess) return e;
  if (!F_in)
    return launch_finish<W_TOK>(partial, T, C, g.S, bias, Gate{a_pre, a_post, a_res}, iters, h_pre, h_post, h_res, st);
  return launch_finish_pre4<W_TOK>(partial, T, C, g.S, bias, Gate{a_pre, a_post, a_res}, iters, h_pre, h_post, h_res, X,
                            F_in, st);
}

hipError_t launch_fast_pre(const void* X, int64_t T, int64_t C, const float* h_pre, void* F_in, hipStream_t st) {
  return launch_pre4(X, T, C, h_pre, F_in, st);
}

hipError_t launch_fast_post_coeffs(const void* X, int64_t T, int64_t C, const float* h_res,
                                   const float* h_post, const void* F, void* Y, const float* phi,
                                   const void* phi_packed, const float* bias, float a_pre, float a_post,
                                   float a_res, int iters, float* h_pre_n, float* h_post_n, float* h_res_n,
                                   void* F_in_n, void* packed, float* partial, hipStream_t st) {
  hipError_t e;
  if (!phi_packed) {
    if ((e = launch_pack(phi, NCOL, nullptr, 0, 4 * C, 24, packed, st)) != hipSuccess) return e;
    phi_packed = packed;
  }
  const Geom g = geom(T, C, 1, TILE);
  SplitArgs A = args(X, T, C, 4 * C, g, phi_packed, partial);
  A.h_res_in = h_res;
  A.h_post_in = h_post;
  A.F = (const uint16_t*)F;
  A.Y = (uint16_t*)Y;
  if ((e = launch_split<true, 3, ROWS_CONTIG>(A, st)) != hipSuccess) return e;
  if (!F_in_n)
    return launch_finish<TILE>(partial, T, C, g.S, bias, Gate{a_pre, a_post, a_res}, iters, h_pre_n, h_post_n,
                               h_res_n, st);
  return launch_finish_pre4<TILE>(partial, T, C, g.S, bias, Gate{a_pre, a_post, a_res}, iters, h_pre_n, h_post_n,
                            h_res_n, Y, F_in_n, st);
}

hipError_t launch_fast_pack(const float* phi, int64_t C, void* packed, hipStream_t st) {
  return launch_pack(phi, NCOL, nullptr, 0, 4 * C, 24, packed, st);
}

// The mHC backward's recompute of the projection, with dH_pre = <dF_in, x_i>
// from the same read of the state: phi's 24 columns padded to 32 (hi and lo
// sharing accumulators), the 4 sums as the partials' extra columns.
int64_t fast_bwd_packed_bytes(int64_t C) { return (int64_t)NS4 * C / 8 * 64 * 16; }
int64_t fast_bwd_partial_bytes(int64_t T, int64_t C) { return part_bytes(T, C, 1, 4, NS4); }

hipError_t launch_fast_bwd_front(const void* X, int64_t T, int64_t C, const float* phi, void* packed,
                                 uint4* phi_rows, float* partial, const void* dF_in, hipStream_t st) {
  hipError_t e = launch_pack(phi, NCOL, nullptr, 0, 4 * C, 32, packed, st, phi_rows);
  if (e != hipSuccess) return e;
  SplitArgs A = args(X, T, C, 4 * C, geom(T, C, 1, W_TOK), packed, partial);
  A.dF = (const uint16_t*)dF_in;
  hipLaunchKernelGGL((proj_wide_kernel<4, ROWS_CONTIG, true, true>), dim3(grid_for(A.nitem)), dim3(STHR), 0, st, A);
  return hipGetLastError();
}

hipError_t launch_fast_xroute_bwd_coeffs(const float* partial, int64_t T, int64_t C, int K, const float* b_act,
                                         float a_post, float a_res, int iters, const float* dh, float* dP, float* g2,
                                         float* red, float* h_res, hipStream_t st) {
  const dim3 grid((unsigned)((T * 16 + 255) / 256)), blk(256);
  const size_t lds = (size_t)iters * 256 * sizeof(float);
  const Gate gt{0.f, a_post, a_res};
  float* dhm = const_cast<float*>(dh);  // read only: the route layouts write no dh
  if (K == 4)
    hipLaunchKernelGGL((bwd_coeff_kernel<W_TOK, 4>), grid, blk, lds, st, partial, T, C, (int)slices(C), b_act, gt,
                       iters, dhm, dP, g2, red, nullptr, h_res);
  else
    hipLaunchKernelGGL((bwd_coeff_kernel<W_TOK, 1>), grid, blk, lds, st, partial, T, C, (int)slices(C), b_act, gt,
                       iters, dhm, dP, g2, red, nullptr, h_res);
  return hipGetLastError();
}

hipError_t launch_fast_xpre_bwd_front(const void* X, int64_t T, int N, int64_t C, const float* phi_pre,
                                      const void* dF_in, void* packed, uint4* phi_rows, float* partial,
                                      hipStream_t st) {
  hipError_t e = launch_pack(phi_pre, N, nullptr, 0, (int64_t)N * C, 16, packed, st, phi_rows);
  if (e != hipSuccess) return e;
  SplitArgs A = args(X, T, C, (int64_t)N * C, geom(T, C, N / 4, W_TOK), packed, partial);
  A.dF = (const uint16_t*)dF_in;
  return launch_wide<2, ROWS_GROUPS, true>(A, st);
}

hipError_t launch_fast_xpre_bwd_coeffs(const float* partial, int64_t T, int N, int64_t C, const float* b_pre,
                                       float a_pre, float* dh_pre, float* dP, float* g2, float* red, float* h_pre,
                                       hipStream_t st) {
  const int64_t threads = T * 16;
  hipLaunchKernelGGL((bwd_xpre_coeff_kernel<2, W_TOK>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     partial, T, C, N, (int)slices(C), b_pre, a_pre, dh_pre, dP, g2, red, h_pre);
  return hipGetLastError();
}

int64_t fast_xroute_partial_bytes(int64_t T, int64_t C, int K) { return part_bytes(T, C, 1, 4); }
int64_t fast_xpre_partial_bytes(int64_t T, int N, int64_t C) { return part_bytes(T, C, N / 4, 2, NS4); }

hipError_t launch_fast_bwd_coeffs(const float* partial, int64_t T, int64_t C, const float* bias, float a_pre,
                                  float a_post, float a_res, int iters, float* dh, float* dP, float* g2,
                                  float* red, float* h_pre, float* h_res, hipStream_t st) {
  const int64_t threads = T * 16;
  hipLaunchKernelGGL((bwd_coeff_kernel<W_TOK, 0, true>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     (size_t)iters * 256 * sizeof(float), st, partial, T, C, (int)slices(C), bias,
                     Gate{a_pre, a_post, a_res}, iters, dh, dP, g2, red, h_pre, h_res);
  return hipGetLastError();
}

// ------------------------------------------------------------------ xHC

XhcFastWs xhc_pre_fast_ws(int64_t T, int N, int64_t C, int m, bool with_router, int dtype) {
  const int ncols = N + (with_router ? N - m : 0);
  if (dtype != 1 || N % 4 != 0 || N > 16 || ncols > 32 || !shape_ok(T, C, N / 4, nb_for(ncols))) return {0, 0};
  const int nb = nb_for(ncols);
  return {(int64_t)N * C / 8 * (nb * 16) * 16, part_bytes(T, C, N / 4, nb)};
}

XhcFastWs xhc_router_fast_ws(int64_t T, int N, int64_t C, int m, int dtype) {
  const int nr = N - m;
  if (dtype != 1 || N % 4 != 0 || N > 16 || nr > 32 || !shape_ok(T, C, N / 4, nb_for(nr))) return {0, 0};
  const int nb = nb_for(nr);
  return {(int64_t)N * C / 8 * (nb * 16) * 16, part_bytes(T, C, N / 4, nb)};
}

// packed column blocks of the active-set projection: up to 32 columns (K <= 4)
// as 4 blocks (2 hi, 2 lo) for the 64-token gathered pass, whose hi and lo
// blocks share accumulators; up to 48 (K <= 8) on 32-token items
static int nb_for_act(int ncols) { return ncols <= 32 ? 4 : (ncols + 7) / 8; }

XhcFastWs xhc_route_fast_ws(int64_t T, int64_t C, int k, int K, int dtype) {
  const int ncols = k * K + k * k;
  if (dtype != 1 || k != 4 || ncols > 48 || !shape_ok(T, C, 1, nb_for_act(ncols))) return {0, 0};
  const int nb = nb_for_act(ncols);
  return {(int64_t)k * C / 8 * (nb * 16) * 16, part_bytes(T, C, 1, nb)};
}

// Full-state projection and finish, on 64-token items (proj_wide_kernel: each
// phi fragment taken from L2 serves 64 tokens). Whether the hi and lo parts of
// phi share accumulators follows from N and m alone, through the column count
// of the pass with both maps (N + N - m): shared unless that pass has 24
// columns (NB = 3, where hi and lo blocks do not pair up; 32 columns need the
// shared form to fit the registers). So the pre map, the router and both
// together add every column in one order and give the same bits.
template <int NB, bool SH>
static hipError_t xhc_full_nb(const void* X, int64_t T, int N, int64_t C, int k, int m, int npre, int nr,
                              const float* b_pre, float a_pre, float* h_pre, float* score, int32_t* idx,
                              const void* packed, float* partial, hipStream_t st) {
  const Geom g = geom(T, C, N / 4, W_TOK);
  const SplitArgs A = args(X, T, C, (int64_t)N * C, g, packed, partial);
  hipLaunchKernelGGL((proj_wide_kernel<NB, ROWS_GROUPS, false, SH>), dim3(grid_for(A.nitem)), dim3(STHR), 0, st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = T * 32;
  hipLaunchKernelGGL((xpre_finish_kernel<NB, W_TOK>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     partial, T, C, N, g.NG * g.S, npre, nr, k, m, b_pre, a_pre, h_pre, score, idx);
  return hipGetLastError();
}

static hipError_t xhc_full_proj(const void* X, int64_t T, int N, int64_t C, int k, int m, int npre, int nr, int nb,
                                 const float* b_pre, float a_pre, float* h_pre, float* score, int32_t* idx,
                                 const void* packed, float* partial, hipStream_t st) {
  const bool shared = nb_for(N + (N - m)) != 3;
#define HC_FULL(NB, SH) \
  xhc_full_nb<NB, SH>(X, T, N, C, k, m, npre, nr, b_pre, a_pre, h_pre, score, idx, packed, partial, st)
  switch (nb) {
    case 2: return shared ? HC_FULL(2, true) : HC_FULL(2, false);
    case 3: return HC_FULL(3, false);
    default: return HC_FULL(4, true);
  }
#undef HC_FULL
}

hipError_t launch_fast_xhc_full(const void* X, int64_t T, int N, int64_t C, int k, int m, const float* phi_pre,
                                const float* b_pre, float a_pre, const float* w_router, float* h_pre, float* score,
                                int32_t* idx, void* F_in, void* packed, float* partial, hipStream_t st) {
  const int npre = phi_pre ? N : 0, nr = w_router ? N - m : 0;
  const int nb = nb_for(npre + nr);
  hipError_t e = phi_pre ? launch_pack(phi_pre, N, w_router, nr, (int64_t)N * C, nb * 8, packed, st)
                         : launch_pack(w_router, nr, nullptr, 0, (int64_t)N * C, nb * 8, packed, st);
  if (e != hipSuccess) return e;
  e = xhc_full_proj(X, T, N, C, k, m, npre, nr, nb, b_pre, a_pre, h_pre, score, idx, packed, partial, st);
  if (e != hipSuccess || !F_in) return e;
  return launch_pre_wide(X, T, N, C, h_pre, F_in, st);
}

// xHC-Flash block entry in one projection pass: the router and the L pre maps
// packed side by side (router first), 64-token items with shared hi/lo
// accumulators, 2 * ceil(columns / 16) packed blocks (at most 80 columns).
static int flash_entry_nb(int N, int m, int L) {
  const int ncols = (N - m) + L * N;
  const int nb = 2 * ((ncols + 15) / 16);
  return nb < 2 ? 2 : nb;
}

XhcFastWs flash_entry_fast_ws(int64_t T, int N, int64_t C, int m, int L, int dtype) {
  if (dtype != 1 || N % 4 != 0 || N > 16 || L < 2 || (N - m) > 32) return {0, 0};
  if ((int64_t)W_TOK * N * C * 2 >= (1ll << 32)) return {0, 0};  // buffer-resource range of a tile
  const int nb = flash_entry_nb(N, m, L);
  if (nb * 8 > PACK_MAXC || !shape_ok(T, C, N / 4, nb)) return {0, 0};
  return {(int64_t)N * C / 8 * (nb * 16) * 16, part_bytes(T, C, N / 4, nb)};
}

template <int NB, int QD>
static hipError_t flash_entry_nb_launch(const SplitArgs& A, const Geom& g, int64_t T, int N, int64_t C, int L, int k,
                                        int m, const float* b_pre, float a_pre, float* h_pre, float* score,
                                        int32_t* idx, const float* partial, hipStream_t st) {
  hipLaunchKernelGGL((proj_wide_kernel<NB, ROWS_GROUPS, false, true, QD>), dim3(grid_for(A.nitem)), dim3(STHR), 0,
                     st, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = T * 32;
  hipLaunchKernelGGL((flash_entry_finish_kernel<NB>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     partial, T, C, N, g.NG * g.S, L, k, m, b_pre, a_pre, h_pre, score, idx);
  return hipGetLastError();
}

hipError_t launch_fast_flash_entry(const void* X, int64_t T, int N, int64_t C, int k, int m, int L,
                                   const float* phi_pre, const float* b_pre, float a_pre, const float* w_router,
                                   float* h_pre, float* score, int32_t* idx, void* packed, float* partial,
                                   hipStream_t st) {
  const int nb = flash_entry_nb(N, m, L);
  const int64_t NC = (int64_t)N * C;
  PackSrcs S{};
  S.p[0] = w_router;
  S.nc[0] = N - m;
  for (int l = 0; l < L; ++l) {
    S.p[1 + l] = phi_pre + (int64_t)l * NC * N;
    S.nc[1 + l] = N;
  }
  S.ns = 1 + L;
  hipLaunchKernelGGL(pack_phi_multi_kernel, dim3((unsigned)(NC / 64)), dim3(256), 0, st, S, nb * 8,
                     (uint16_t*)packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const Geom g = geom(T, C, N / 4, W_TOK);
  const SplitArgs A = args(X, T, C, NC, g, packed, partial);
#define HC_FE(NB, QD) flash_entry_nb_launch<NB, QD>(A, g, T, N, C, L, k, m, b_pre, a_pre, h_pre, score, idx, partial, st)
  switch (nb) {
    case 2: return HC_FE(2, 4);
    case 4: return HC_FE(4, 4);
    case 6: return HC_FE(6, 4);
    case 8: return HC_FE(8, 2);
    default: return HC_FE(10, 2);
  }
#undef HC_FE
}

// ------------------------------------------------------- xHC chained step
// The full-state maps of sublayer l + 1 ([pre N | router N - m], packed as
// NB = 4 blocks with shared hi/lo accumulators, 64-token items) over the state
// route l has just written, from two parts: the carry, partials over the rows
// route l left unchanged (formed by the dense read of the call before, which
// leaves route l's active rows out), and the active rows themselves after the
// mix, grouped by stream so that each pair tile multiplies one stream's phi
// rows (ROWS_PAIRS). The state is then read once per sublayer: by the dense
// read, which also forms the next carry.
constexpr int CH_NB = 4;
static int chain_ntile(int64_t T, int k, int N) { return (int)((T * k + W_TOK - 1) / W_TOK) + N; }

bool xhc_chain_supported(int dtype, int64_t T, int N, int64_t C, int k, int m) {
  const int nc = N + (N - m);
  return dtype == 1 && N == 16 && k == 4 && m >= 1 && m <= k && nc > 24 && nc <= 32 && C % 512 == 0 && T >= 1 &&
         T * k < (1ll << 30) && shape_ok(T, C, N / 4, CH_NB) && (int64_t)W_TOK * N * C * 2 < (1ll << 32) &&
         (int64_t)chain_ntile(T, k, N) * slices(C / 4) * W_TOK * (CH_NB * 8 + 1) * 4 < (1ll << 31);
}

static int sort_blocks(int64_t T) { return (int)((T + SORT_THR - 1) / SORT_THR); }

// the carry: the partials, then the packed maps they were formed with
int64_t xhc_chain_carry_part_bytes(int64_t T, int N, int64_t C) {
  return (part_bytes(T, C, N / 4, CH_NB) + 255) / 256 * 256;
}
int64_t xhc_chain_carry_bytes(int64_t T, int N, int64_t C) {
  return xhc_chain_carry_part_bytes(T, N, C) + (int64_t)N * C / 8 * (CH_NB * 16) * 16;
}

XhcChainWs xhc_chain_ws(int64_t T, int N, int64_t C, int k) {
  const int ntile = chain_ntile(T, k, N);
  XhcChainWs w;
  w.packed = (int64_t)N * C / 8 * (CH_NB * 16) * 16;
  w.pair_part = (int64_t)ntile * slices(C / 4) * W_TOK * (CH_NB * 8 + 1) * 4;
  w.ptok = (int64_t)ntile * W_TOK * 4;
  w.pos = T * k * 4;
  w.tile_off = (int64_t)(N + 1) * 4;
  w.sort = 2ll * sort_blocks(T) * N * 4;
  return w;
}

hipError_t launch_fast_pre_wide(const void* X, int64_t T, int N, int64_t C, const float* h_pre, void* F_in,
                               hipStream_t st) {
  return launch_pre_wide(X, T, N, C, h_pre, F_in, st);
}

hipError_t launch_fast_xhc_pack_full(const float* phi_pre, const float* w_router, int N, int m, int64_t C,
                                     void* packed, hipStream_t st) {
  return launch_pack(phi_pre, N, w_router, N - m, (int64_t)N * C, CH_NB * 8, packed, st);
}

hipError_t launch_fast_xhc_dense(const void* X, int64_t T, int N, int64_t C, const float* h_pre, const int32_t* idx,
                                 const void* packed, void* F_in, float* carry, hipStream_t st) {
  const Geom g = geom(T, C, N / 4, W_TOK);
  SplitArgs A = args(X, T, C, (int64_t)N * C, g, packed, carry);
  A.hd = h_pre;
  A.Fd = (uint16_t*)F_in;
  A.idx = idx;
  A.kidx = 4;
  A.nstreams = N;
  hipLaunchKernelGGL((proj_wide_kernel<CH_NB, ROWS_DENSE, false, true, 2>), dim3(grid_for(A.nitem)), dim3(STHR), 0,
                     st, A);
  return hipGetLastError();
}

hipError_t launch_fast_xhc_chain_maps(const void* X, int64_t T, int N, int64_t C, int k, int m,
                                      const int32_t* idx_prev, const void* packed, const float* carry,
                                      const float* b_pre, float a_pre, float* h_pre, float* score, int32_t* idx,
                                      int32_t* ptok, int32_t* tile_off, int32_t* pos, int32_t* sortw,
                                      float* pair_part, hipStream_t st) {
  const int ntile = chain_ntile(T, k, N);
  const int G = sort_blocks(T);
  int32_t* cnt = sortw;
  int32_t* base = sortw + (int64_t)G * N;
  hipLaunchKernelGGL(pair_count_kernel, dim3(G), dim3(SORT_THR), 0, st, idx_prev, T, k, N, cnt);
  hipLaunchKernelGGL(pair_scan_kernel, dim3(1), dim3(SORT_THR), 0, st, (const int32_t*)cnt, G, N, ntile, tile_off, base,
                     ptok);
  hipLaunchKernelGGL(pair_place_kernel, dim3(G), dim3(SORT_THR), 0, st, idx_prev, T, k, N, (const int32_t*)base, ptok,
                     pos);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t Cq = C / 4;  // the quarter rows that stand in for a pair's 4 streams
  const int ps = (int)slices(Cq);
  const Geom gp{1, ps, ntile * ps};
  SplitArgs A = args(X, T, Cq, (int64_t)N * C, gp, packed, pair_part);
  A.ptok = ptok;
  A.tile_off = tile_off;
  A.nstreams = N;
  A.sq = C;
  hipLaunchKernelGGL((proj_wide_kernel<CH_NB, ROWS_PAIRS, false, true, 4>), dim3(grid_balanced(A.nitem)), dim3(STHR),
                     0, st, A);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const Geom g = geom(T, C, N / 4, W_TOK);
  const int64_t threads = T * 32;
  hipLaunchKernelGGL((xpre_finish_kernel<CH_NB, W_TOK, true>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, carry, T, C, N, g.NG * g.S, N, N - m, k, m, b_pre, a_pre, h_pre, score, idx,
                     (const float*)pair_part, (const int32_t*)pos, k, ps);
  return hipGetLastError();
}

// Streaming copy of n16 16-byte words: 4 per thread, all loads issued before
// the stores, nontemporal both ways (the probe of the streaming rate).
__global__ __launch_bounds__(256) void copy_probe_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  u32x4_t v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int64_t i = base + k * 256;
    i = i < n16 ? i : n16 - 1;
    v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + i));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t i = base + k * 256;
    if (i < n16) __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4_t*>(dst + i));
  }
}

hipError_t launch_copy_probe(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)((n16 + 1023) / 1024)), dim3(256), 0, st,
                     (const uint4*)src, (uint4*)dst, n16);
  return hipGetLastError();
}

bool fast_mix_supported(int dtype, int k, int K, int64_t C, const void* X, const void* Wb) {
  return dtype == 1 && k == 4 && K >= 1 && K <= 8 && C % 8 == 0 && a16(X) && a16(Wb);
}

hipError_t launch_fast_mix(void* X, int64_t T, int N, int64_t C, const int32_t* idx, const float* H_res,
                           const float* H_post, const void* Wb, int K, hipStream_t st, const void* Wb2, int j0) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T * (C / 8) + 255) / 256)), blk(256);
  uint16_t* x = (uint16_t*)X;
  const uint16_t* w = (const uint16_t*)Wb;
  const uint16_t* w2 = (const uint16_t*)Wb2;
  if (!Wb2) j0 = K;
  if (Wb2) {
    switch (K) {
      case 1: hipLaunchKernelGGL((mix4_kernel<1, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 2: hipLaunchKernelGGL((mix4_kernel<2, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 3: hipLaunchKernelGGL((mix4_kernel<3, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 4: hipLaunchKernelGGL((mix4_kernel<4, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 5: hipLaunchKernelGGL((mix4_kernel<5, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 6: hipLaunchKernelGGL((mix4_kernel<6, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 7: hipLaunchKernelGGL((mix4_kernel<7, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      default: hipLaunchKernelGGL((mix4_kernel<8, true>), grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
    }
  } else {
    switch (K) {
      case 1: hipLaunchKernelGGL(mix4_kernel<1>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 2: hipLaunchKernelGGL(mix4_kernel<2>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 3: hipLaunchKernelGGL(mix4_kernel<3>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 4: hipLaunchKernelGGL(mix4_kernel<4>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 5: hipLaunchKernelGGL(mix4_kernel<5>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 6: hipLaunchKernelGGL(mix4_kernel<6>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      case 7: hipLaunchKernelGGL(mix4_kernel<7>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
      default: hipLaunchKernelGGL(mix4_kernel<8>, grid, blk, 0, st, x, T, N, C, idx, H_res, H_post, w, w2, j0); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_fast_xhc_active(const void* X, int64_t T, int N, int64_t C, const int32_t* idx, int K,
                                  const float* phi_act, const float* b_act, float a_post, float a_res, int iters,
                                  float* Hp, float* Hr, void* packed, float* partial, hipStream_t st,
                                  uint4* phi_rows, bool nt_rows) {
  const int ncols = 4 * K + 16;
  const int nb = nb_for_act(ncols);
  hipError_t e;
  if (ncols <= 32) {
    e = launch_pack(phi_act, ncols, nullptr, 0, 4 * C, nb * 8, packed, st, phi_rows);
  } else {  // more columns than the two-source pack holds (no row form: the backward takes K <= 4)
    PackSrcs S{};
    S.p[0] = phi_act;
    S.nc[0] = ncols;
    S.ns = 1;
    hipLaunchKernelGGL(pack_phi_multi_kernel, dim3((unsigned)(4 * C / 64)), dim3(256), 0, st, S, nb * 8,
                       (uint16_t*)packed);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  // up to 32 columns: 64-token items (each phi fragment from L2 serves 64
  // tokens); wider: 32-token items
  const bool wide = ncols <= 32;
  const Geom g = geom(T, C, 1, wide ? W_TOK : TILE);
  SplitArgs A = args(X, T, C, (int64_t)N * C, g, packed, partial);
  A.idx = idx;
  A.kidx = 4;
  A.nstreams = N;
  // nt_rows: nontemporal loads of the gathered rows, for a caller whose next
  // pass gains less from finding them in the last-level cache than those loads
  // gain here (the forward mix with K > 1 components, which reads as many bytes
  // of them as of the rows: projection + mix 195 against 202 us at K = 4, N =
  // 16, C = 4096, T = 8192; at K = 1, 158 against 168 us the other way).
  if (wide && nt_rows) {
    hipLaunchKernelGGL((proj_wide_kernel<4, ROWS_GATHER, false, true, 4, true>), dim3(grid_for(A.nitem)), dim3(STHR), 0,
                       st, A);
    e = hipGetLastError();
  } else if (wide) {
    hipLaunchKernelGGL((proj_wide_kernel<4, ROWS_GATHER, false, true, 4>), dim3(grid_for(A.nitem)), dim3(STHR), 0, st,
                       A);
    e = hipGetLastError();
  } else {
    e = launch_split_gather(nb, A, st);
  }
  if (e != hipSuccess) return e;
  const int64_t threads = T * 16;
  const dim3 grid((unsigned)((threads + 255) / 256)), blk(256);
#define HC_XRF(NB, TT) \
  hipLaunchKernelGGL((xroute_finish_kernel<NB, TT>), grid, blk, 0, st, partial, T, C, g.S, K, b_act, a_post, a_res, \
                     iters, Hp, Hr)
  switch (nb) {
    case 4: HC_XRF(4, W_TOK); break;
    case 5: HC_XRF(5, TILE); break;
    default: HC_XRF(6, TILE); break;
  }
#undef HC_XRF
  return hipGetLastError();
}

}  // namespace hc
