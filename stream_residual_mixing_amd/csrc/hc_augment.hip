// Temporal feature augmentation for the configuration of the xHC summary
// (K_r = 4: F_out and causal depthwise convs with kappa = 4, 8, 12), in two
// passes over F_out.
//
// [xHC] temporal feature augmentation: g_j[t, c] = sum_{s < kappa_j}
// w_j[c, s] F[t - kappa_j + 1 + s, c] with zeros before each sequence start,
// then Gram-Schmidt of a_0 = F, a_1..a_3 = g_1..g_3:
//   v_0 = a_0,  v_j = a_j - sum_{i<j} (<a_j, v_i> / <v_i, v_i>) v_i.
// The pages name the modified form, which equals this one in exact arithmetic.
// Every inner product here is a combination of the entries of the 4x4 Gram
// matrix G = [<a_i, a_j>] of the token: writing v_j = sum_k B[j][k] a_k,
//   <a_j, v_i> = sum_k B[i][k] G[k][j],  <v_i, v_i> = B_i^T G B_i,
// so the first pass only accumulates G (per token, per 512-channel slice) and
// the second pass rebuilds B (in float64) and writes V = B A. The full-C
// reductions then need no workgroup to hold a token's whole row. (In float32
// this matches float64 modified Gram-Schmidt to about 3e-8 relative L2 on
// data of this shape, as the float32 modified form does.) Tokens whose Gram
// matrix shows a component close to the span of the earlier ones, where this
// form loses accuracy faster than the modified one, are then redone by a third
// pass that runs the modified form literally.
//
// The Gram pass works one position per lane (below); the apply pass, whose
// stores must run along the channels, works one channel pair per thread: a
// workgroup of 256 threads x 2 channels = a 512-channel slice, over a strip of
// 36 consecutive tokens of one sequence; each thread keeps its channels' 24 conv
// taps and the last 12 rows of F in registers, so F is read once per pass (plus
// an 11-row halo per strip).
#include <type_traits>

#include "hc_device.h"
#include "hc_fast.h"

namespace hc {

namespace {

constexpr int K1 = 4, K2 = 8, K3 = 12;
constexpr int ATT = 3 * K3;         // tokens per strip (a multiple of the ring length)
// Channels per thread of the apply pass (a workgroup of 256 threads covers 512):
// 2 rather than 4 halves the registers for taps and the ring, for more waves
// per SIMD.
constexpr int CH_A = 2;
constexpr int NG10 = 10;            // upper triangle of the 4x4 Gram matrix
constexpr int NB6 = 6;              // strictly lower part of B

// A row of CH channels of one thread, as loaded (converted to float when used).
template <typename TF, int CH>
struct RawRow;
template <>
struct RawRow<float, 4> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void get(float o[4]) const { o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w; }
};
template <>
struct RawRow<float, 2> {
  float2 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ void get(float o[2]) const { o[0] = v.x; o[1] = v.y; }
};
template <>
struct RawRow<bf16_t, 4> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void get(float o[4]) const {
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};
template <>
struct RawRow<bf16_t, 2> {
  uint32_t v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ void get(float o[2]) const {
    o[0] = __uint_as_float(v << 16); o[1] = __uint_as_float(v & 0xffff0000u);
  }
};
// Buffer resource over [base, base + bytes): stores whose offset falls outside
// are dropped by the hardware.
constexpr unsigned BUF_DW3 = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;  // any offset >= the range is dropped

// CH channels of one thread at byte offset off of a buffer resource
template <typename TV, int CH>
__device__ __forceinline__ void stb(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  if constexpr (std::is_same<TV, float>::value && CH == 4)
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])}, r, off,
        0, 0);
  else if constexpr (std::is_same<TV, float>::value)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[0]), __float_as_uint(v[1])}, r, off, 0, 0);
  else if constexpr (CH == 4)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf2_hw(v[0], v[1]), pack_bf2_hw(v[2], v[3])}, r, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b32(pack_bf2_hw(v[0], v[1]), r, off, 0, 0);
}

// Where a workgroup works: sequence b, token positions [p0, p1), channels
// c0..c0+CH-1 of its thread (cok: inside C; C % 4 == 0).
struct Place {
  int64_t b, p0, p1, c0;
  bool cok;
};
template <int CH>
__device__ __forceinline__ Place place(int64_t S, int64_t C, int nstrip, int nslice) {
  const int slice = (int)(blockIdx.x % nslice);
  const int64_t rest = blockIdx.x / nslice;
  const int64_t strip = rest % nstrip;
  Place pl;
  pl.b = rest / nstrip;
  pl.p0 = strip * ATT;
  pl.p1 = pl.p0 + ATT < S ? pl.p0 + ATT : S;
  const int64_t c = (int64_t)slice * (256 * CH) + threadIdx.x * CH;
  pl.cok = c < C;
  pl.c0 = pl.cok ? c : 0;
  return pl;
}

// The taps of the three convs for channels c0..c0+CH-1 (w: [C, 4] | [C, 8] | [C, 12]).
template <int CH>
struct Taps {
  float w1[K1][CH], w2[K2][CH], w3[K3][CH];
};
template <int CH>
__device__ __forceinline__ void load_taps(const float* __restrict__ w, int64_t C, int64_t c0, Taps<CH>& tp) {
#pragma unroll
  for (int ch = 0; ch < CH; ++ch) {
    const float* p1 = w + (c0 + ch) * K1;
    const float* p2 = w + K1 * C + (c0 + ch) * K2;
    const float* p3 = w + (K1 + K2) * C + (c0 + ch) * K3;
#pragma unroll
    for (int s = 0; s < K1; ++s) tp.w1[s][ch] = p1[s];
#pragma unroll
    for (int s = 0; s < K2; ++s) tp.w2[s][ch] = p2[s];
#pragma unroll
    for (int s = 0; s < K3; ++s) tp.w3[s][ch] = p3[s];
  }
}

// Walks the strip's ATT tokens in order with the last 12 rows of F (this
// thread's channels) in a register ring: row p sits in slot (p - p0) mod 12 (p0
// is a multiple of 12), so with the walk unrolled by 12 every slot index is a
// compile-time constant. Rows are loaded PF tokens ahead into a small queue
// (slot (p - p0) mod PF) as loaded, and converted into the ring once the token
// PF - 1 places earlier is done (the ring slot they take still holds row
// p - 11, the oldest tap of that token). The walk always covers ATT tokens, past
// the strip end too (rows clamped to the sequence, results discarded by the
// caller), and every load is unconditional: the compiler can then count the
// loads in flight exactly and waits only for the row it needs. fn(p, a)
// receives a[0..3][ch] = F, g1, g2, g3 of token p (zeros past C).
constexpr int PF = 4;  // rows in flight (divides 12; 4 measured faster than 6 or 12)

template <bool FC, int CH, typename TF, typename Fn>  // FC: C is a multiple of the slice width
__device__ __forceinline__ void walk_strip(const TF* __restrict__ F, int64_t S, int64_t C, const Place& pl,
                                           const Taps<CH>& tp, Fn fn) {
  static_assert(K3 % PF == 0 && ATT % K3 == 0, "ring and queue slots must be compile-time constants");
  const TF* base = F + pl.b * S * C + pl.c0;
  auto at = [&](int64_t p) __attribute__((always_inline)) { return base + (p < 0 ? 0 : (p < S ? p : S - 1)) * C; };
  float ring[K3][CH];
  RawRow<TF, CH> q[PF];
  {
    // rows p0-11 .. p0-1 in slots 1..11 and p0 in slot 0, all loads issued first;
    // rows before the sequence start are zeros (a mask, not a branch)
    RawRow<TF, CH> r0[K3];
#pragma unroll
    for (int sl = 0; sl < K3; ++sl) r0[sl].load(at(sl == 0 ? pl.p0 : pl.p0 - K3 + sl));
#pragma unroll
    for (int d = 1; d < PF; ++d) q[d].load(at(pl.p0 + d));
#pragma unroll
    for (int sl = 0; sl < K3; ++sl) {
      r0[sl].get(ring[sl]);
      const uint32_t keep = (sl == 0 || pl.p0 - K3 + sl >= 0) ? 0xffffffffu : 0u;
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) ring[sl][ch] = __uint_as_float(__float_as_uint(ring[sl][ch]) & keep);
    }
  }
  for (int blk = 0; blk < ATT / K3; ++blk) {
#pragma unroll
    for (int u = 0; u < K3; ++u) {
      const int64_t p = pl.p0 + blk * K3 + u;
      q[u % PF].load(at(p + PF));  // the slot of row p, already in the ring
      float a[4][CH];
#pragma unroll
      for (int ch = 0; ch < CH; ++ch) {
        // tap s of a kappa-wide conv reads row p - kappa + 1 + s, in slot (u + 1 + s + 12 - kappa) mod 12
        float g1 = 0.f, g2 = 0.f, g3 = 0.f;
#pragma unroll
        for (int s = 0; s < K1; ++s) g1 += tp.w1[s][ch] * ring[(u + 1 + s + K3 - K1) % K3][ch];
#pragma unroll
        for (int s = 0; s < K2; ++s) g2 += tp.w2[s][ch] * ring[(u + 1 + s + K3 - K2) % K3][ch];
#pragma unroll
        for (int s = 0; s < K3; ++s) g3 += tp.w3[s][ch] * ring[(u + 1 + s) % K3][ch];
        const bool cok = FC || pl.cok;
        a[0][ch] = cok ? ring[u][ch] : 0.f;
        a[1][ch] = cok ? g1 : 0.f;
        a[2][ch] = cok ? g2 : 0.f;
        a[3][ch] = cok ? g3 : 0.f;
      }
      fn(p, a);
      q[(u + 1) % PF].get(ring[(u + 1) % K3]);
    }
  }
}

// Pass 1: partial Gram matrices gram[t][slice][10] (upper triangle, row-major),
// one position per lane. A workgroup of 1024 threads (16 waves) takes a block of
// GT = 256 consecutive positions of one sequence (lane l of every wave: positions
// 4l..4l+3 of the block) and a slice of GCS channels, in chunks of 64 channels
// staged through LDS as float columns [channel][row], row 0 = 11 positions before
// the block (zeros before the sequence start and past C). Wave w takes channels
// w, w + 16, w + 32, w + 48 of each chunk: the channel is the same across the
// wave, so its 24 taps come by scalar loads, and each lane adds its 4 positions'
// 10 products over its channels with no exchange between lanes. The 16 waves'
// sums are added through LDS at the end, in wave order.
constexpr int GW = 1024;               // threads per workgroup
constexpr int GT = 256;                // positions per workgroup (4 per lane)
constexpr int GCK = 64;                // channels per LDS chunk
constexpr int GCS = 8 * GCK;           // channels per workgroup
constexpr int GROWS = GT + K3 - 1;     // staged rows of a chunk
// Column of one channel: 16-byte blocks of 4 rows; block b of channel c sits at
// block position b ^ (c / 4 mod 16), so the staging writes (16 lanes, 16 channel
// groups, one row) and the window reads (64 lanes, 64 consecutive blocks) both
// hit distinct banks. 80 blocks = 320 rows cover every swizzled position.
constexpr int GRS = 320;
static_assert(((GROWS + 3) / 4 + 3 + 15) / 16 * 16 * 4 <= GRS, "swizzled blocks fit the column");
constexpr int GUNITS = GROWS * (GCK / 4);  // staging units of 4 channels x 1 row per chunk
constexpr int GUPT = (GUNITS + GW - 1) / GW;

__device__ __forceinline__ int gswz(int cl, int row) {  // LDS float index of (channel cl, row)
  return cl * GRS + ((((row >> 2) ^ ((cl >> 2) & 15))) << 2) + (row & 3);
}

template <typename TF>
__global__ __launch_bounds__(GW) void aug_gram_kernel(const TF* __restrict__ F, int64_t S, int64_t C,
                                                      const float* __restrict__ w, int nblk, int nslice,
                                                      float* __restrict__ gram) {
  __shared__ __attribute__((aligned(16))) float tile[GCK * GRS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slice = (int)(blockIdx.x % nslice);
  const int64_t rest = blockIdx.x / nslice;
  const int64_t b = rest / nblk, p0 = (rest % nblk) * GT;
  const int64_t cbase = (int64_t)slice * GCS;
  const TF* Fb = F + b * S * C;
  // staging: unit u = (row u / 16, channels 4 (u % 16) .. +3 of the chunk)
  RawRow<TF, 4> st[GUPT];
  auto stage_load = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GUPT; ++i) {
      const int u = i * GW + tid;
      const int r = (u < GUNITS ? u : GUNITS - 1) >> 4;
      const int64_t pos = p0 - (K3 - 1) + r;
      const int64_t c = cbase + (int64_t)k * GCK + (u & 15) * 4;
      st[i].load(Fb + (pos < 0 ? 0 : (pos < S ? pos : S - 1)) * C + (c < C ? c : 0));
    }
  };
  auto stage_store = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GUPT; ++i) {
      const int u = i * GW + tid;
      if (u < GUNITS) {
        const int r = u >> 4, g = u & 15;
        const int64_t pos = p0 - (K3 - 1) + r;
        const bool ok = pos >= 0 && cbase + (int64_t)k * GCK + g * 4 < C;
        float v[4];
        st[i].get(v);
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[gswz(g * 4 + e, r)] = ok ? v[e] : 0.f;
      }
    }
  };
  float acc[4][NG10];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < NG10; ++q) acc[j][q] = 0.f;
  const int nchunk = (int)((C - cbase + GCK - 1) / GCK < GCS / GCK ? (C - cbase + GCK - 1) / GCK : GCS / GCK);
  stage_load(0);
  for (int k = 0; k < nchunk; ++k) {
    __syncthreads();  // the previous chunk's reads are done
    stage_store(k);
    __syncthreads();
    if (k + 1 < nchunk) stage_load(k + 1);
#pragma unroll
    for (int cw = 0; cw < GCK / 16; ++cw) {
      const int cl = wv + 16 * cw;  // channel within the chunk (uniform over the wave)
      int64_t c = cbase + (int64_t)k * GCK + cl;
      c = c < C ? c : 0;
      const float* t1 = w + c * K1;
      const float* t2 = w + K1 * C + c * K2;
      const float* t3 = w + (K1 + K2) * C + c * K3;
      float x[16];  // rows 4l .. 4l+15 of this channel
#pragma unroll
      for (int bi = 0; bi < 4; ++bi) {
        const float4 q4 = *reinterpret_cast<const float4*>(&tile[gswz(cl, 4 * (lane + bi))]);
        x[4 * bi] = q4.x;
        x[4 * bi + 1] = q4.y;
        x[4 * bi + 2] = q4.z;
        x[4 * bi + 3] = q4.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // position 4l + j of the block is row 4l + j + 11
        float a[4];
        a[0] = x[j + K3 - 1];
        float g1 = 0.f, g2 = 0.f, g3 = 0.f;
#pragma unroll
        for (int s = 0; s < K1; ++s) g1 += t1[s] * x[j + K3 - K1 + s];
#pragma unroll
        for (int s = 0; s < K2; ++s) g2 += t2[s] * x[j + K3 - K2 + s];
#pragma unroll
        for (int s = 0; s < K3; ++s) g3 += t3[s] * x[j + s];
        a[1] = g1;
        a[2] = g2;
        a[3] = g3;
        int q = 0;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
#pragma unroll
          for (int j2 = i2; j2 < 4; ++j2) acc[j][q++] += a[i2] * a[j2];
      }
    }
  }
  // the 16 waves' sums, in two rounds of 5 entries: [wave][entry][position]
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 5; ++q) tile[(wv * 5 + q) * GT + 4 * lane + j] = acc[j][half * 5 + q];
    __syncthreads();
    for (int i = tid; i < 5 * GT; i += GW) {
      const int q = i / GT, pp = i - q * GT;
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < GW / 64; ++ww) v += tile[(ww * 5 + q) * GT + pp];
      const int64_t pos = p0 + pp;
      if (pos < S) gram[((b * S + pos) * nslice + slice) * NG10 + half * 5 + q] = v;
    }
  }
}

// The coefficients of token t's components from its Gram partials: v_j =
// sum_k B[j][k] a_k, with <a_j, v_i> = B_i . G[:, j] and <v_i, v_i> = B_i^T G B_i
// (the slices added in order, all in float64). vv[j] = <v_j, v_j>, gd[j] = G[j][j].
__device__ __forceinline__ void gram_to_b(const float* __restrict__ gram, int64_t t, int nslice, double Bm[4][4],
                                          double vv[4], double gd[4]) {
  double G[4][4];
  double gs[NG10];
#pragma unroll
  for (int k = 0; k < NG10; ++k) gs[k] = 0.0;
  for (int sl = 0; sl < nslice; ++sl) {
    const float* gp = gram + (t * nslice + sl) * NG10;
#pragma unroll
    for (int k = 0; k < NG10; ++k) gs[k] += (double)gp[k];
  }
  int q = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = i; j < 4; ++j) {
      G[i][j] = gs[q];
      G[j][i] = gs[q];
      ++q;
    }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) Bm[i][j] = i == j ? 1.0 : 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < j; ++i) {
      double num = 0.0;
#pragma unroll
      for (int k = 0; k <= i; ++k) num += Bm[i][k] * G[k][j];
      const double cji = num / vv[i];
#pragma unroll
      for (int k = 0; k <= i; ++k) Bm[j][k] -= cji * Bm[i][k];
    }
    double qf = 0.0;
#pragma unroll
    for (int k = 0; k <= j; ++k)
#pragma unroll
      for (int l = 0; l <= j; ++l) qf += Bm[j][k] * G[k][l] * Bm[j][l];
    vv[j] = qf;
    gd[j] = G[j][j];
  }
}

// The Gram form loses accuracy as a component approaches the span of the earlier
// ones: its error grows with the square of the condition number, the modified
// form's with the condition number. vv_j / G_jj is the squared sine of the angle
// between a_j and that span; a token with any of these below GS_MIN_SIN2 (an angle
// under 30 degrees), or not finite, is redone by the literal modified form
// (aug_mgs_fix_kernel). On the workload's data the smallest value is near 1.
constexpr double GS_MIN_SIN2 = 0.25;

__device__ __forceinline__ bool gram_ill_conditioned(const double vv[4], const double gd[4]) {
  bool bad = false;
#pragma unroll
  for (int j = 1; j < 4; ++j) bad |= !(vv[j] >= GS_MIN_SIN2 * gd[j]);  // NaN counts as bad
  return bad;
}

// Pass 2: thread i < strip length builds B of token p0 + i from its Gram matrix
// into LDS; then V[t, j] = a_j + sum_{k<j} B[j][k] a_k.
template <bool FC, typename TF, typename TV>
__global__ __launch_bounds__(256) void aug_apply_kernel(const TF* __restrict__ F, int64_t S, int64_t C,
                                                        const float* __restrict__ w, int nstrip, int nslice_a,
                                                        int nslice, const float* __restrict__ gram,
                                                        TV* __restrict__ V) {
  __shared__ float Bs[ATT][NB6];
  const Place pl = place<CH_A>(S, C, nstrip, nslice_a);
  if ((int64_t)threadIdx.x < pl.p1 - pl.p0) {
    const int64_t t = pl.b * S + pl.p0 + threadIdx.x;
    double Bm[4][4], vv[4], gd[4];
    gram_to_b(gram, t, nslice, Bm, vv, gd);
    float* out = Bs[threadIdx.x];
    out[0] = (float)Bm[1][0];
    out[1] = (float)Bm[2][0];
    out[2] = (float)Bm[2][1];
    out[3] = (float)Bm[3][0];
    out[4] = (float)Bm[3][1];
    out[5] = (float)Bm[3][2];
  }
  __syncthreads();
  Taps<CH_A> tp;
  load_taps(w, C, pl.c0, tp);
  // V rows of this sequence through a buffer resource: a store of a token past
  // the strip or of channels past C gets an out-of-range offset and is dropped
  // (no branch around a store)
  const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
      V + pl.b * S * 4 * C, 0, (uint32_t)(S * 4 * C * (int64_t)sizeof(TV)), BUF_DW3);
  walk_strip<FC, CH_A, TF>(F, S, C, pl, tp, [&](int64_t p, const float (&a)[4][CH_A]) __attribute__((always_inline)) {
    const float* bq = Bs[p - pl.p0];  // rows past the strip hold stale values (their stores are dropped)
    const bool ok = (FC || pl.cok) && p < pl.p1;
    auto off = [&](int j) __attribute__((always_inline)) {
      return ok ? (uint32_t)(((p * 4 + j) * C + pl.c0) * (int64_t)sizeof(TV)) : OOB;
    };
    float v[CH_A];
    stb<TV, CH_A>(vres, off(0), a[0]);
#pragma unroll
    for (int ch = 0; ch < CH_A; ++ch) v[ch] = a[1][ch] + bq[0] * a[0][ch];
    stb<TV, CH_A>(vres, off(1), v);
#pragma unroll
    for (int ch = 0; ch < CH_A; ++ch) v[ch] = a[2][ch] + bq[1] * a[0][ch] + bq[2] * a[1][ch];
    stb<TV, CH_A>(vres, off(2), v);
#pragma unroll
    for (int ch = 0; ch < CH_A; ++ch) v[ch] = a[3][ch] + bq[3] * a[0][ch] + bq[4] * a[1][ch] + bq[5] * a[2][ch];
    stb<TV, CH_A>(vres, off(3), v);
  });
}


// Pass 3, for the tokens gram_ill_conditioned() flags: the modified Gram-Schmidt
// of the xHC summary (temporal feature augmentation) taken literally in float32,
// overwriting what pass 2 wrote for them. A workgroup of 256 threads checks 64
// consecutive tokens (wave 0, one token per lane) and then works through the
// flagged ones in token order, all 256 threads over the channels. A channel's
// components are recomputed in every round instead of being stored, so any C
// fits; each round forms the same float32 values by the same fused steps:
//   round 1: n0 = <v0, v0>, d_j0 = <a_j, v0> (v0 = a0)
//   round 2: v1 = a1 - c10 v0; n1 = <v1, v1>, d_j1 = <a_j - c_j0 v0, v1> (j = 2, 3)
//   round 3: v2 = (a2 - c20 v0) - c21 v1; n2 = <v2, v2>, d32 = <(a3 - c30 v0) - c31 v1, v2>
//   round 4: v3 = ((a3 - c30 v0) - c31 v1) - c32 v2; store v0..v3
// with c_ji = d_ji / n_i. Sums are float32, per thread over its channels, then
// over the lanes and the 4 waves in a fixed order.
constexpr int FIX_TOK = 64;

template <typename TF>
__device__ __forceinline__ void conv_at(const TF* __restrict__ Fseq, int64_t pos, int64_t C, int64_t c,
                                        const float* __restrict__ w, float a[4]) {
  a[0] = Elem<TF>::ld(Fseq + pos * C + c);
  const int kap[3] = {K1, K2, K3};
  const float* wj = w;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    float g = 0.f;
    for (int s = 0; s < kap[j]; ++s) {
      const int64_t src = pos - kap[j] + 1 + s;
      if (src >= 0) g = __fmaf_rn(wj[c * kap[j] + s], Elem<TF>::ld(Fseq + src * C + c), g);
    }
    a[j + 1] = g;
    wj += kap[j] * C;
  }
}

template <int NS>
__device__ __forceinline__ void block_sums(float (&v)[NS], float (*red)[4]) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NS; ++k) v[k] = wave_sum(v[k]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int k = 0; k < NS; ++k) red[wid][k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < NS; ++k) v[k] = ((red[0][k] + red[1][k]) + red[2][k]) + red[3][k];
}

template <typename TF, typename TV>
__global__ __launch_bounds__(256) void aug_mgs_fix_kernel(const TF* __restrict__ F, int64_t S, int64_t T, int64_t C,
                                                          const float* __restrict__ w, int nslice,
                                                          const float* __restrict__ gram, TV* __restrict__ V) {
  __shared__ unsigned long long flags;
  __shared__ float red[4][4];
  const int64_t t0 = (int64_t)blockIdx.x * FIX_TOK;
  if (threadIdx.x < 64) {
    const int64_t t = t0 + threadIdx.x;
    bool bad = false;
    if (t < T) {
      double Bm[4][4], vv[4], gd[4];
      gram_to_b(gram, t, nslice, Bm, vv, gd);
      bad = gram_ill_conditioned(vv, gd);
    }
    const unsigned long long m = __ballot(bad);
    if (threadIdx.x == 0) flags = m;
  }
  __syncthreads();
  unsigned long long m = flags;
  while (m) {
    const int i = __builtin_ctzll(m);
    m &= m - 1;
    const int64_t t = t0 + i;
    const int64_t pos = t % S;
    const TF* Fseq = F + (t - pos) * C;
    float a[4];
    float r1[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t c = threadIdx.x; c < C; c += 256) {
      conv_at(Fseq, pos, C, c, w, a);
      r1[0] = __fmaf_rn(a[0], a[0], r1[0]);
      r1[1] = __fmaf_rn(a[1], a[0], r1[1]);
      r1[2] = __fmaf_rn(a[2], a[0], r1[2]);
      r1[3] = __fmaf_rn(a[3], a[0], r1[3]);
    }
    block_sums<4>(r1, red);
    const float c10 = r1[1] / r1[0], c20 = r1[2] / r1[0], c30 = r1[3] / r1[0];
    float r2[3] = {0.f, 0.f, 0.f};
    for (int64_t c = threadIdx.x; c < C; c += 256) {
      conv_at(Fseq, pos, C, c, w, a);
      const float v1 = __fmaf_rn(-c10, a[0], a[1]);
      const float u2 = __fmaf_rn(-c20, a[0], a[2]);
      const float u3 = __fmaf_rn(-c30, a[0], a[3]);
      r2[0] = __fmaf_rn(v1, v1, r2[0]);
      r2[1] = __fmaf_rn(u2, v1, r2[1]);
      r2[2] = __fmaf_rn(u3, v1, r2[2]);
    }
    block_sums<3>(r2, red);
    const float c21 = r2[1] / r2[0], c31 = r2[2] / r2[0];
    float r3[2] = {0.f, 0.f};
    for (int64_t c = threadIdx.x; c < C; c += 256) {
      conv_at(Fseq, pos, C, c, w, a);
      const float v1 = __fmaf_rn(-c10, a[0], a[1]);
      const float v2 = __fmaf_rn(-c21, v1, __fmaf_rn(-c20, a[0], a[2]));
      const float u3 = __fmaf_rn(-c31, v1, __fmaf_rn(-c30, a[0], a[3]));
      r3[0] = __fmaf_rn(v2, v2, r3[0]);
      r3[1] = __fmaf_rn(u3, v2, r3[1]);
    }
    block_sums<2>(r3, red);
    const float c32 = r3[1] / r3[0];
    TV* out = V + t * 4 * C;
    for (int64_t c = threadIdx.x; c < C; c += 256) {
      conv_at(Fseq, pos, C, c, w, a);
      const float v1 = __fmaf_rn(-c10, a[0], a[1]);
      const float v2 = __fmaf_rn(-c21, v1, __fmaf_rn(-c20, a[0], a[2]));
      const float v3 = __fmaf_rn(-c32, v2, __fmaf_rn(-c31, v1, __fmaf_rn(-c30, a[0], a[3])));
      Elem<TV>::st(out + c, a[0]);
      Elem<TV>::st(out + C + c, v1);
      Elem<TV>::st(out + 2 * C + c, v2);
      Elem<TV>::st(out + 3 * C + c, v3);
    }
  }
}

template <typename TF, typename TV>
hipError_t launch_aug(const void* F, int64_t B, int64_t S, int64_t C, const float* w, void* V, float* gram,
                      hipStream_t st) {
  const int nstrip = (int)((S + ATT - 1) / ATT);
  const int nblk = (int)((S + GT - 1) / GT);
  const int nslice = (int)((C + GCS - 1) / GCS);
  const int nslice_a = (int)((C + 256 * CH_A - 1) / (256 * CH_A));
  const dim3 grid((unsigned)(B * nblk * nslice)), grid_a((unsigned)(B * nstrip * nslice_a)), blk(256);
  hipLaunchKernelGGL(aug_gram_kernel<TF>, grid, dim3(GW), 0, st, (const TF*)F, S, C, w, nblk, nslice, gram);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (C % (256 * CH_A) == 0)
    hipLaunchKernelGGL((aug_apply_kernel<true, TF, TV>), grid_a, blk, 0, st, (const TF*)F, S, C, w, nstrip, nslice_a,
                       nslice, (const float*)gram, (TV*)V);
  else
    hipLaunchKernelGGL((aug_apply_kernel<false, TF, TV>), grid_a, blk, 0, st, (const TF*)F, S, C, w, nstrip,
                       nslice_a, nslice, (const float*)gram, (TV*)V);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t T = B * S;
  hipLaunchKernelGGL((aug_mgs_fix_kernel<TF, TV>), dim3((unsigned)((T + FIX_TOK - 1) / FIX_TOK)), blk, 0, st,
                     (const TF*)F, S, T, C, w, nslice, (const float*)gram, (TV*)V);
  return hipGetLastError();
}

}  // namespace

bool fast_augment_supported(int dtype, int vdtype, int64_t S, int64_t C, const int* kappa, int r, const void* F,
                            const void* V) {
  if (r != 3 || kappa[0] != K1 || kappa[1] != K2 || kappa[2] != K3 || C % 4 != 0) return false;
  // one sequence's V addressed with 32-bit buffer offsets
  if (S * 4 * C * (vdtype == 0 ? 4 : 2) >= (1ll << 31)) return false;
  const uintptr_t fa = dtype == 0 ? 16 : 8, va = vdtype == 0 ? 16 : 8;
  return ((uintptr_t)F % fa) == 0 && ((uintptr_t)V % va) == 0;
}

int64_t fast_augment_workspace_bytes(int64_t B, int64_t S, int64_t C) {
  return B * S * ((C + GCS - 1) / GCS) * NG10 * 4;
}

hipError_t launch_fast_augment(int dtype, int vdtype, const void* F, int64_t B, int64_t S, int64_t C,
                               const float* w, void* V, float* gram, hipStream_t st) {
  if (dtype == 0 && vdtype == 0) return launch_aug<float, float>(F, B, S, C, w, V, gram, st);
  if (dtype == 0) return launch_aug<float, bf16_t>(F, B, S, C, w, V, gram, st);
  if (vdtype == 0) return launch_aug<bf16_t, float>(F, B, S, C, w, V, gram, st);
  return launch_aug<bf16_t, bf16_t>(F, B, S, C, w, V, gram, st);
}

}  // namespace hc
