// mHC sublayer backward for n = 4 bfloat16 streams on gfx950.
//
// "mHC: Manifold-Constrained Hyper-Connections" (paper notes), 4.3.1: the
// backward of the Eq. 14-15 kernel holds two products over the same x, and the
// Sinkhorn-Knopp backward recomputes the iterates on chip and walks the
// iterations; 4.3 also recomputes the mHC kernels' intermediates in the
// backward instead of keeping them. Two stages, in the order a training step
// meets them:
//  post stage (before the sublayer function's backward, which needs dF_out):
//    bwd_post_kernel: dF_out = H_post dX_next (H_post the forward's) and per
//    token dh[4:24] = [dH_post | dH_res] (sums over the channels);
//  main stage (once dF_in is known):
//  1. phi packed in two forms (projection and dP phi^T operands) and the
//     projection partials of X by the forward's kernel (hc_fused.hip), with
//     the partial sums of dh[0:4] = dH_pre = <dF_in, x_i> formed from the same
//     tiles of X (dF_in read beside them);
//  2. bwd_coeff_kernel (hc_fused.hip, beside the forward finish whose floats it
//     recomputes): dH_pre summed into dh, gates and Sinkhorn backward -> dP,
//     g2, sums over groups of 16 tokens, and the forward's h_pre and h_res;
//  3. bwd_dx_kernel: dX = H_res^T dX_next + H_pre dF_in + dP phi^T + g2 x, the
//     dP phi^T product on MFMA, and from the same tiles of x the dphi partials
//     vec(x)^T dP over groups of token tiles on MFMA (the tokens are the K
//     dimension);
//  4. bwd_sums_kernel: the group partials of dphi and the sums of db and dalpha
//     added in a fixed order.
#include "hc.h"
#include "hc_device.h"
#include "hc_fast.h"

namespace hc {
namespace {

typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));

constexpr int BS = 4;     // streams
constexpr int BCOL = 24;  // n*n + 2n columns: [pre 4 | post 4 | res 16]
constexpr int DPS = 32;   // floats per dP row (columns 24..31 zero)
constexpr int RED = 36;   // floats per row of the sums over 16 tokens: dz [32] | 3 gate sums | 0

// Row modes of the passes: which stream row of a token slot i (of 4) is, and
// which phi rows it multiplies.
//  BM_MHC:   the n = 4 state: row t*4 + i, phi rows i*C + c;
//  BM_ROUTE: the xHC active set: row t*N + idx[t*4 + i] (slot order), phi rows
//            i*C + c (phi_act is in slot order); updated in place;
//  BM_PRE:   stream group g = blockIdx.z of an N-stream state: row t*N + 4g + i,
//            phi rows (4g + i)*C + c.
constexpr int BM_MHC = 0, BM_ROUTE = 1, BM_PRE = 2;

// stream index of slot i of token t (loaded from idx for BM_ROUTE and clamped
// into [0, N), so no index reaches outside the token's row)
template <int BM>
__device__ __forceinline__ void slot_streams(const int32_t* idx, int64_t t, int N, int (&s)[4]) {
  if constexpr (BM == BM_ROUTE) {
    const int4 v = reinterpret_cast<const int4*>(idx)[t];
    const int w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = w[i] < 0 ? 0 : (w[i] >= N ? N - 1 : w[i]);
  } else {
    const int g0 = BM == BM_PRE ? 4 * (int)blockIdx.z : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = g0 + i;
  }
}

__device__ __forceinline__ bf8_t bf8(const uint4& q) { return __builtin_bit_cast(bf8_t, q); }

__device__ __forceinline__ uint4 ld_nt16(const uint16_t* p) {
  const u4_t v = __builtin_nontemporal_load(reinterpret_cast<const u4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void unpack_bf8(const uint4& q, float v[8]) {
  v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
  v[4] = __uint_as_float(q.z << 16); v[5] = __uint_as_float(q.z & 0xffff0000u);
  v[6] = __uint_as_float(q.w << 16); v[7] = __uint_as_float(q.w & 0xffff0000u);
}

// v = hi + lo with hi = bf16(v) and lo = bf16(v - hi) (v - hi is exact in float32),
// each as 8 packed bfloat16: about 16 significant bits of v.
__device__ __forceinline__ void split_bf8(const float v[8], uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    h[k] = pack_bf2_hw(v[2 * k], v[2 * k + 1]);
    l[k] = pack_bf2_hw(v[2 * k] - __uint_as_float(h[k] << 16), v[2 * k + 1] - __uint_as_float(h[k] & 0xffff0000u));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ------------------------------------------------------- per-token sums

// One 256-thread workgroup per token t (post stage), over the 4 slots of the
// row mode (the n = 4 state, or the xHC active set) with K write-back
// components Wb_j (the n = 4 state and K = 1: F_out):
//   dWb_j = sum_i H_post[i, j] dX_next_i     (K = 1: bfloat16, rounded once;
//                                             K = 4: float32, for the
//                                             augmentation backward)
//   dh[off + i*K + j]          = dH_post[i, j] = <dX_next_i, Wb_j>
//   dh[off + 4K + 4i + k]      = dH_res[i][k]  = <dX_next_i, x_k>
// (dh rows of dhs floats; h_post [T, 4K] as the forward formed it). Thread tid
// takes the 8-channel chunks tid, tid + 256, ...; the threads' sums are added
// by a butterfly in each wave and then the 4 waves in order.
template <int BM, int K>
__global__ __launch_bounds__(256) void bwd_post_kernel(const uint16_t* __restrict__ X,
                                                       const uint16_t* __restrict__ dXn,
                                                       const uint16_t* __restrict__ Wb, int64_t C, int N,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ h_post, float* __restrict__ dh,
                                                       int dhs, int off, void* __restrict__ dWb) {
  constexpr int NA = 4 * K + 16;  // sums per token
  __shared__ float wsum[4][NA];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  float hpost[4][K];  // hpost[i][j] = H_post[i, j]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < K; ++j) hpost[i][j] = h_post[t * 4 * K + i * K + j];
  float acc[NA];
#pragma unroll
  for (int k = 0; k < NA; ++k) acc[k] = 0.f;
  const int64_t nch = C / 8;
  int sl[4];
  slot_streams<BM>(idx, t, N, sl);
  for (int64_t j = tid; j < nch; j += 256) {
    const int64_t c = j * 8;
    uint4 xq[BS], dq[BS], wq[K];
#pragma unroll
    for (int i = 0; i < BS; ++i) {
      xq[i] = ld_nt16(X + (t * N + sl[i]) * C + c);
      dq[i] = ld_nt16(dXn + (t * N + sl[i]) * C + c);
    }
#pragma unroll
    for (int q = 0; q < K; ++q) wq[q] = ld_nt16(Wb + (t * K + q) * C + c);
    float x[BS][8], d[BS][8], f[K][8];
#pragma unroll
    for (int i = 0; i < BS; ++i) {
      unpack_bf8(xq[i], x[i]);
      unpack_bf8(dq[i], d[i]);
    }
#pragma unroll
    for (int q = 0; q < K; ++q) unpack_bf8(wq[q], f[q]);
#pragma unroll
    for (int q = 0; q < K; ++q) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = hpost[0][q] * d[0][e] + hpost[1][q] * d[1][e] + hpost[2][q] * d[2][e] + hpost[3][q] * d[3][e];
      if constexpr (K == 1) {
        __builtin_nontemporal_store(u4_t{pack_bf2_hw(o[0], o[1]), pack_bf2_hw(o[2], o[3]), pack_bf2_hw(o[4], o[5]),
                                         pack_bf2_hw(o[6], o[7])},
                                    reinterpret_cast<u4_t*>(reinterpret_cast<uint16_t*>(dWb) + t * C + c));
      } else {
        float* dst = reinterpret_cast<float*>(dWb) + (t * K + q) * C + c;
        __builtin_nontemporal_store(f4_t{o[0], o[1], o[2], o[3]}, reinterpret_cast<f4_t*>(dst));
        __builtin_nontemporal_store(f4_t{o[4], o[5], o[6], o[7]}, reinterpret_cast<f4_t*>(dst) + 1);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int i = 0; i < BS; ++i) {
#pragma unroll
        for (int q = 0; q < K; ++q) acc[i * K + q] += d[i][e] * f[q][e];
#pragma unroll
        for (int k = 0; k < BS; ++k) acc[4 * K + 4 * i + k] += d[i][e] * x[k][e];
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NA; ++k) acc[k] = wave_sum(acc[k]);
  if ((tid & 63) == 0) {
#pragma unroll
    for (int k = 0; k < NA; ++k) wsum[tid >> 6][k] = acc[k];
  }
  __syncthreads();
  if (tid < NA) dh[t * dhs + off + tid] = ((wsum[0][tid] + wsum[1][tid]) + wsum[2][tid]) + wsum[3][tid];
}

// ------------------------------------------------------------------- dX

constexpr int FT = 32;          // tokens per tile
constexpr int FCH = 128;        // channels per chunk
constexpr int FROW = FCH * 2;   // bytes per (stream, token) row of the state tile
constexpr int DPT = FT + 8;     // bfloat16 per column of the transposed dP tile (80 bytes)

// Byte offset of (stream i, token m, channel c) in the state tile. The 16-byte
// block c >> 3 of a row sits at block (c >> 3) ^ (((m >> 3) & 3) << 1): the
// A-fragment reads (16 consecutive channels of tokens m, m + 8, m + 16, m + 24)
// then fall in distinct banks.
__device__ __forceinline__ int xoff(int i, int m, int c) {
  return (i * FT + m) * FROW + (((c >> 3) ^ (((m >> 3) & 3) << 1)) << 4) + (c & 7) * 2;
}


constexpr unsigned BUFW3 = 0x00020000u;  // buffer-resource word 3 (raw, 32-bit data)
constexpr uint32_t OOBW = 0x80000000u;   // an offset no range reaches: the access is dropped
constexpr int XT = 32;        // tokens per item
constexpr int XCH = 128;      // channels per item
constexpr int PRJ = XCH + 4;  // floats per (stream, token) row of the product tile in LDS
static_assert(XT == FT && XCH == FCH, "the dphi MFMAs take the dX tile's state rows");

// dX over items of 32 tokens x 128 channels x the 4 slots of the row mode, 512
// threads. The grid is (chunk, group[, stream group for BM_PRE]): workgroup
// (c, j) keeps the channel chunk c and walks the token tiles j, j + J, ...
// (J = gridDim.y), so its phi fragments load once. Everything a tile needs
// from memory is loaded one tile ahead into a second register set: thread
// (token tid >> 4, channels (tid & 15) * 8) takes its 16-byte pieces of x and
// dX_next in the 4 slots and of dF_in; threads tid < 192 one 16-byte piece of
// the tile's coefficients [h_res 16 | h_pre 4 | g2 | 0 0 0] and threads
// tid < 256 one of its dP rows, both staged in LDS at the start of the tile.
// Per tile:
//  * MFMA phase: wave w forms dP phi^T for slot w >> 1, the four 16-channel
//    blocks (w & 1) * 4 .. + 3 and both 16-token blocks
//    (v_mfma_f32_16x16x32_bf16; A = the tokens' dP rows split hi/lo, B = the
//    channels' phi rows hi/lo; hi*hi + hi*lo + lo*hi into one float32
//    accumulator) into the LDS product tile; then the next tile's loads are
//    issued, and the same wave adds the tile's x^T dP to its dphi
//    accumulators for the same slot and channel blocks and both 16-column
//    blocks of dP, with the tokens as K (A = x^T, one channel and 8 tokens a
//    lane, read from the state tile the threads also stage in LDS; B = dP
//    transposed and split hi/lo, zero past T; D += A B_hi + A B_lo);
//  * streaming phase, slot j:
//      BM_MHC:   dX_j = sum_i H_res[i, j] dX_next_i + H_pre[j] dF_in + (dP phi^T)_j + g2 x_j
//      BM_ROUTE: dX_j = sum_i H_res[i, j] dX_next_i + (dP phi^T)_j + g2 x_j, written over
//                dX_next's row (the same memory)
//      BM_PRE:   dX_j += H_pre[j] dF_in + (dP phi^T)_j + g2 x_j (dX_next is dX)
//    rounded once to bfloat16 and stored.
// Rows past T and channels past C are computed on clamped addresses and not
// stored. After the last tile each workgroup writes its dphi partials,
//   part[blockIdx.y][R][k] = sum over its tiles of x[t, slot, c] dP[t, k]   (k < ncol)
// with R the phi row of the slot's channel c, added over the groups later in a
// fixed order. In place is safe: a thread reads its (token, channels) of dX_next one
// tile before it writes the same elements, and no other thread touches them.
constexpr int CFR = 24;  // floats per token of the staged coefficients
constexpr int DPR = 36;  // floats per token row of the staged dP tile (padded)

template <int BM>
__global__ __launch_bounds__(512) void bwd_dx_kernel(const uint16_t* __restrict__ X, const uint16_t* dXn,
                                                     const uint16_t* __restrict__ dFi, int64_t T, int64_t C, int N,
                                                     const int32_t* __restrict__ idx, const float* __restrict__ h_pre,
                                                     const float* __restrict__ h_res, const float* __restrict__ dP,
                                                     const float* __restrict__ g2, const uint4* __restrict__ phi_rows,
                                                     uint16_t* dX, int ncol, int64_t nrows,
                                                     float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float prj[BS * XT * PRJ];
  __shared__ __attribute__((aligned(16))) float cf[XT * CFR];
  __shared__ __attribute__((aligned(16))) float dpt[XT * DPR];
  // the dphi MFMAs' tiles: the state (swizzled) and dP transposed, hi and lo
  __shared__ __attribute__((aligned(16))) unsigned char xt[BS * FT * FROW];
  __shared__ __attribute__((aligned(16))) uint16_t dph[2 * DPS * DPT];  // [hi | lo][column][token]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t chunk = blockIdx.x;
  const int64_t J = gridDim.y, ntile = (T + XT - 1) / XT;
  const int m = tid >> 4, c8 = (tid & 15) * 8;
  const int64_t c = chunk * XCH + c8;
  const bool cok = c < C;
  const int64_t cl = cok ? c : C - 8;
  const int si = wave >> 1, cb0 = (wave & 1) * 4;
  const int tau = lane & 15, q = lane >> 4;
  const int g0 = BM == BM_PRE ? 4 * (int)blockIdx.z : 0;  // first phi row group (BM_PRE)
  // staging roles: coefficient piece (token tid / 6, piece tid % 6), dP piece
  // (token (tid & 255) >> 3, piece tid & 7)
  const int ctok = tid < 192 ? tid / 6 : 0, cpc = tid < 192 ? tid - 6 * ctok : 0;
  const int dtok = (tid & 255) >> 3, dpc = tid & 7;

  constexpr int PNB = BM == BM_PRE ? 1 : 2;  // dP column blocks of 16 (the pre mode has N <= 16 columns)
  f4_t pacc[4][PNB];                        // dphi: [channel block][dP column block]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int nb = 0; nb < PNB; ++nb) pacc[cb][nb] = f4_t{0.f, 0.f, 0.f, 0.f};
  // The phi fragments of the dP phi^T product (this wave's stream and channel
  // blocks, hi and lo) stay for the whole kernel: in registers, except the hi
  // parts of the mHC and route modes, which go to LDS (each wave its own 4 KB)
  // to make room for their H_res product beside the dphi accumulators.
  constexpr bool PHL = BM != BM_PRE;
  __shared__ __attribute__((aligned(16))) uint4 phl[PHL ? 8 * 4 * 64 : 1];
  uint4 bh[PHL ? 1 : 4], bl[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    int64_t ch = chunk * XCH + (cb0 + cb) * 16 + tau;
    ch = ch < C ? ch : C - 1;
    const uint4* pr = phi_rows + ((int64_t)(g0 + si) * C + ch) * 8;
    if constexpr (PHL) phl[(wave * 4 + cb) * 64 + lane] = pr[q];
    else bh[cb] = pr[q];
    bl[cb] = pr[4 + q];
  }

  struct In {
    uint4 xq[BS], dq[BS], fq;
    float4 cv, dv;
    int sl[4];  // the slots' streams
  };
  auto load = [&](int64_t tl, In& in) __attribute__((always_inline)) {
    const int64_t t = tl * XT + m;
    const int64_t tc = t < T ? t : T - 1;
    slot_streams<BM>(idx, tc, N, in.sl);
    // Buffer loads over the tile's token rows (rows past T read as zeros): a
    // 32-bit offset per thread and, for the fixed slots of the mHC and pre
    // modes, each slot's offset in a scalar register, where 64-bit addresses per
    // row held registers the fused dphi products need.
    const int64_t r0 = tl * XT;
    const int64_t nrow = T - r0 < XT ? T - r0 : XT;
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(X) + r0 * N * C, 0, (uint32_t)(nrow * N * C * 2), BUFW3);
    const __amdgpu_buffer_rsrc_t dr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(dXn) + r0 * N * C, 0, (uint32_t)(nrow * N * C * 2), BUFW3);
#pragma unroll
    for (int i = 0; i < BS; ++i) {
      uint32_t vo, so;
      if constexpr (BM == BM_ROUTE) {
        vo = (uint32_t)((((int64_t)m * N + in.sl[i]) * C + cl) * 2);
        so = 0;
      } else {
        vo = (uint32_t)(((int64_t)m * N * C + cl) * 2);
        so = (uint32_t)((int64_t)(g0 + i) * C * 2);
      }
      const u4_t a = __builtin_amdgcn_raw_buffer_load_b128(xr, vo, so, 2);
      const u4_t b = __builtin_amdgcn_raw_buffer_load_b128(dr, vo, so, 2);
      in.xq[i] = make_uint4(a.x, a.y, a.z, a.w);
      in.dq[i] = make_uint4(b.x, b.y, b.z, b.w);
    }
    if constexpr (BM != BM_ROUTE) {
      const __amdgpu_buffer_rsrc_t fr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(dFi) + r0 * C, 0, (uint32_t)(nrow * C * 2), BUFW3);
      const u4_t f = __builtin_amdgcn_raw_buffer_load_b128(fr, (uint32_t)(((int64_t)m * C + cl) * 2), 0, 2);
      in.fq = make_uint4(f.x, f.y, f.z, f.w);
    }
    int64_t t1 = tl * XT + ctok;
    t1 = t1 < T ? t1 : T - 1;
    if (cpc < 4) {
      if constexpr (BM == BM_PRE) in.cv = make_float4(0.f, 0.f, 0.f, 0.f);
      else in.cv = reinterpret_cast<const float4*>(h_res + t1 * 16)[cpc];
    } else if (cpc == 4) {
      if constexpr (BM == BM_ROUTE) in.cv = make_float4(0.f, 0.f, 0.f, 0.f);
      else in.cv = *reinterpret_cast<const float4*>(h_pre + t1 * (BM == BM_PRE ? N : 4) + g0);
    } else {
      in.cv = make_float4(g2[t1], 0.f, 0.f, 0.f);
    }
    int64_t t2 = tl * XT + dtok;
    t2 = t2 < T ? t2 : T - 1;
    in.dv = reinterpret_cast<const float4*>(dP + t2 * DPS)[dpc];
  };
  // one tile: returns false after the last
  auto step = [&](int64_t& tl, In& cur, In& nxt) __attribute__((always_inline)) {
    if (tid < 192) *reinterpret_cast<float4*>(cf + ctok * CFR + cpc * 4) = cur.cv;
#pragma unroll
    for (int i = 0; i < BS; ++i) *reinterpret_cast<uint4*>(xt + xoff(i, m, c8)) = cur.xq[i];
    if (tid < 256) *reinterpret_cast<float4*>(dpt + dtok * DPR + dpc * 4) = cur.dv;
    if (tid < 256) {
      const bool pok = tl * XT + dtok < T;
      const float v[4] = {cur.dv.x, cur.dv.y, cur.dv.z, cur.dv.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float vk = pok ? v[k] : 0.f;
        const uint32_t h = f2bf(vk);
        const uint32_t l = f2bf(vk - bf2f(h));
        dph[(dpc * 4 + k) * DPT + dtok] = (uint16_t)h;
        dph[(DPS + dpc * 4 + k) * DPT + dtok] = (uint16_t)l;
      }
    }
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const float4* pa = reinterpret_cast<const float4*>(dpt + (tb * 16 + tau) * DPR + q * 8);
      const float4 a0 = pa[0], a1 = pa[1];
      const float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      uint4 ah, al;
      split_bf8(v, ah, al);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        uint4 bhc;
        if constexpr (PHL) bhc = phl[(wave * 4 + cb) * 64 + lane];
        else bhc = bh[cb];
        f4_t acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8(ah), bf8(bhc), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8(ah), bf8(bl[cb]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8(al), bf8(bhc), acc, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) prj[(si * XT + tb * 16 + q * 4 + e) * PRJ + (cb0 + cb) * 16 + tau] = acc[e];
      }
    }
    const int64_t nt = tl + J;
    if (nt < ntile) load(nt, nxt);
    {
      uint4 ph[PNB], pl[PNB];
#pragma unroll
      for (int nb = 0; nb < PNB; ++nb) {
        ph[nb] = *reinterpret_cast<const uint4*>(dph + (nb * 16 + tau) * DPT + q * 8);
        pl[nb] = *reinterpret_cast<const uint4*>(dph + (DPS + nb * 16 + tau) * DPT + q * 8);
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int chl = (cb0 + cb) * 16 + tau;
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t lo16 = *reinterpret_cast<const uint16_t*>(xt + xoff(si, q * 8 + 2 * k, chl));
          const uint32_t hi16 = *reinterpret_cast<const uint16_t*>(xt + xoff(si, q * 8 + 2 * k + 1, chl));
          w[k] = lo16 | (hi16 << 16);
        }
        const uint4 xa = make_uint4(w[0], w[1], w[2], w[3]);
#pragma unroll
        for (int nb = 0; nb < PNB; ++nb) {
          pacc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8(xa), bf8(ph[nb]), pacc[cb][nb], 0, 0, 0);
          pacc[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf8(xa), bf8(pl[nb]), pacc[cb][nb], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    // the token's staged coefficients [h_res 16 | h_pre 4 | g2 ...]: H[i][j] =
    // h_res[t, i, j], read from LDS where each output slot j uses them
    const float* cft = cf + m * CFR;
    const float4 hp4 = reinterpret_cast<const float4*>(cft)[4], g4 = reinterpret_cast<const float4*>(cft)[5];
    const float hp[4] = {hp4.x, hp4.y, hp4.z, hp4.w};
    // dX_next and dF_in stay packed (bfloat16 pairs) and each value is widened
    // where it is used, rather than all 40 at once; likewise h_res is read from
    // LDS a column at a time (these registers are what the dphi accumulators need)
    auto dn = [&](int i, int e) __attribute__((always_inline)) {
      const uint32_t w = e < 2 ? cur.dq[i].x : (e < 4 ? cur.dq[i].y : (e < 6 ? cur.dq[i].z : cur.dq[i].w));
      return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    };
    auto fn = [&](int e) __attribute__((always_inline)) {
      const uint32_t w = e < 2 ? cur.fq.x : (e < 4 ? cur.fq.y : (e < 6 ? cur.fq.z : cur.fq.w));
      return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
    };
    const int64_t t = tl * XT + m;
    const bool ok = t < T && cok;
    const int64_t nrw = T - tl * XT < XT ? T - tl * XT : XT;
    const __amdgpu_buffer_rsrc_t xw =
        __builtin_amdgcn_make_buffer_rsrc(dX + tl * XT * N * C, 0, (uint32_t)(nrw * N * C * 2), BUFW3);
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const float4* pj = reinterpret_cast<const float4*>(prj + (j * XT + m) * PRJ + c8);
      const float4 p0 = pj[0], p1 = pj[1];
      const float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
      float xj[8], o[8];
      unpack_bf8(*reinterpret_cast<const uint4*>(xt + xoff(j, m, c8)), xj);
      const float H0 = cft[j], H1 = cft[4 + j], H2 = cft[8 + j], H3 = cft[12 + j];  // column j
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v;
        if constexpr (BM == BM_PRE) v = dn(j, e) + hp[j] * fn(e);
        else v = H0 * dn(0, e) + H1 * dn(1, e) + H2 * dn(2, e) + H3 * dn(3, e);
        if constexpr (BM == BM_MHC) v += hp[j] * fn(e);
        o[e] = v + p[e] + g4.x * xj[e];
      }
      // through a buffer resource over the tile's rows: past T or C the offset is
      // out of range and the store is dropped (nontemporal)
      uint32_t off = OOBW;
      if (ok) {
        if constexpr (BM == BM_ROUTE) off = (uint32_t)((((int64_t)m * N + cur.sl[j]) * C + c) * 2);
        else off = (uint32_t)((((int64_t)m * N + g0 + j) * C + c) * 2);
      }
      __builtin_amdgcn_raw_buffer_store_b128(u4_t{pack_bf2_hw(o[0], o[1]), pack_bf2_hw(o[2], o[3]),
                                                  pack_bf2_hw(o[4], o[5]), pack_bf2_hw(o[6], o[7])},
                                             xw, off, 0, 2);
    }
    __syncthreads();  // the LDS tiles are rewritten by the next tile
    tl = nt;
    return nt < ntile;
  };
  int64_t tl = blockIdx.y;
  In a, b;
  load(tl, a);
  while (step(tl, a, b) && step(tl, b, a)) {
  }
  float* out = part + (int64_t)blockIdx.y * nrows * ncol;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int nb = 0; nb < PNB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t ch = chunk * XCH + (cb0 + cb) * 16 + q * 4 + e;
        const int col = nb * 16 + tau;
        if (ch < C && col < ncol) out[((int64_t)(g0 + si) * C + ch) * ncol + col] = pacc[cb][nb][e];
      }
}

// The final sums in one launch. Workgroups [0, nbp): dphi, the G group
// partials added in group order, one thread per entry. Workgroup nbp + k:
// column k of the sums over groups of 16 tokens [nrow][28] added over the
// groups: dbias[k] for k < nb, then dalpha[k - nb] = column a0 + (k - nb) for
// the next workgroups; each thread the rows tid, tid + 256, ... in order, then
// a tree in LDS.
__global__ __launch_bounds__(256) void bwd_sums_kernel(const float* __restrict__ part, int64_t n, int G, int nbp,
                                                       float* __restrict__ dphi, const float* __restrict__ red,
                                                       int64_t nrow, int nb, float* __restrict__ dbias, int a0,
                                                       float* __restrict__ dalpha) {
  const int tid = threadIdx.x;
  if ((int)blockIdx.x < nbp) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + tid;
    if (g >= n) return;
    float s = 0.f;
    for (int k = 0; k < G; ++k) s += part[(int64_t)k * n + g];
    dphi[g] = s;
    return;
  }
  __shared__ float sm[256];
  const int k = (int)blockIdx.x - nbp;
  const int colk = k < nb ? k : a0 + (k - nb);
  float v = 0.f;
  for (int64_t t = tid; t < nrow; t += 256) v += red[t * RED + colk];
  sm[tid] = v;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) sm[tid] += sm[tid + h];
    __syncthreads();
  }
  if (tid == 0) {
    if (k < nb) dbias[k] = sm[0];
    else dalpha[k - nb] = sm[0];
  }
}

// ------------------------------------------ temporal augmentation backward

// Backward of xhc_augment for r = 3 causal depthwise convs of sizes 4, 8, 12
// ([xHC] temporal feature augmentation): components u_0 = F_out, u_j = conv_j
// (F_out), V = modified Gram-Schmidt of [u_0..u_3]; upstream dV [T, 4, C]
// float32. Per token every vector involved lies in the span of u_0..u_3 and
// dV_0..dV_3, so the Gram-Schmidt backward needs only the Gram matrix G = U U^T
// and M = dV U^T (26 sums over the channels): dU_i = sum_q P[i][q] dV_q +
// sum_k Q[i][k] u_k with 4 x 4 matrices P, Q from G and M. Four launches:
//  1. aug_bwd_gram_kernel: a workgroup takes 256 channels (one per thread) and
//     a strip of tokens; each thread walks the strip with the last 12 rows of
//     F_out in registers and the next 4 tokens' loads in flight, forms u_1..u_3
//     and the 26 products, the wave sums them over its 64 channels in one
//     reduce-scatter, and every 32 tokens the 4 waves' sums are added in LDS
//     and stored as part [channel group][26][T];
//  2. aug_bwd_coef_kernel: the channel groups' sums added in order per token,
//     then one thread per token walks the Gram-Schmidt steps, recomputed, in
//     reverse in float64 on the 4-coefficient representation: P, Q [T][32];
//  3. aug_bwd_walk_kernel: one thread per channel walks a strip backwards (plus
//     the 11 tokens after it, within the sequence), the strip's P, Q staged in
//     LDS: dU from P, Q, the ring of the next 11 tokens' dU_j, dF_out[t] =
//     dU_0[t] + sum_j sum_d w_j[kappa_j - 1 - d] dU_j[t + d] (the conv's
//     transpose), and the tap gradients dw_j[s] += dU_j[t] F_out[t - kappa_j +
//     1 + s] summed over the strip's tokens into wpart [strip][24][C];
//  4. aug_bwd_wsum_kernel: the strips' tap sums added in strip order.
// Both walks keep F_out's rows as loaded and mask, per token, the window
// positions before the token's sequence start, so a sequence boundary inside a
// strip needs no reload.
constexpr int AB_STRIP = 128;  // tokens per strip (AB_STRIP2 when that still gives enough workgroups)
constexpr int AB_STRIP2 = 256;
constexpr int AB_GRP = 32;     // tokens per cross-wave sum of the Gram pass
constexpr int AB_PF = 4;       // tokens per load group (the next group is in flight)
constexpr int AB_NV = 26;      // sums per token: G (10, upper triangle) | M (16, M[j][i] = <dV_j, u_i>)
constexpr int AB_K1 = 4, AB_K2 = 8, AB_K3 = 12, AB_TAPS = AB_K1 + AB_K2 + AB_K3;
static_assert(AB_STRIP % AB_GRP == 0 && AB_STRIP2 % AB_GRP == 0 && AB_GRP % AB_PF == 0,
              "strip, group and load group nest");

// Workgroup barrier ordering LDS only: global loads in flight stay in flight
// (a full __syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// element at byte offset `off` (per lane, 32 bits) of the row starting at `row`
// (uniform): the address splits into a scalar base and a 32-bit lane offset
template <typename TF>
__device__ __forceinline__ float ab_ldo(const TF* row, uint32_t off) {
  const TF* p = reinterpret_cast<const TF*>(reinterpret_cast<const char*>(row) + off);
  if constexpr (sizeof(TF) == 2) return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  else return *reinterpret_cast<const float*>(p);
}

template <typename TF>
__device__ __forceinline__ float ab_ld(const TF* p) {
  if constexpr (sizeof(TF) == 2) return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  else return *reinterpret_cast<const float*>(p);
}

// win[s] = F_out[t - 11 + s] as loaded; ts = t's position in its sequence.
// Positions before the sequence start read as zero.
__device__ __forceinline__ void ab_mask(const float (&win)[12], int64_t ts, float (&wm)[12]) {
#pragma unroll
  for (int s = 0; s < 12; ++s) wm[s] = s + ts >= 11 ? win[s] : 0.f;
}

// the three convs at the current token from the masked window wm[0..11] = F_out[t-11..t]
__device__ __forceinline__ void ab_convs(const float (&w)[AB_TAPS], const float (&wm)[12], float (&u)[4]) {
  u[0] = wm[11];
  float a = 0.f, b = 0.f, c = 0.f;
#pragma unroll
  for (int s = 0; s < AB_K1; ++s) a += w[s] * wm[12 - AB_K1 + s];
#pragma unroll
  for (int s = 0; s < AB_K2; ++s) b += w[AB_K1 + s] * wm[12 - AB_K2 + s];
#pragma unroll
  for (int s = 0; s < AB_K3; ++s) c += w[AB_K1 + AB_K2 + s] * wm[12 - AB_K3 + s];
  u[1] = a;
  u[2] = b;
  u[3] = c;
}

// taps of channel c (conv_w = [C, 4] | [C, 8] | [C, 12])
__device__ __forceinline__ void ab_taps(const float* __restrict__ conv_w, int64_t C, int64_t c, float (&w)[AB_TAPS]) {
#pragma unroll
  for (int s = 0; s < AB_K1; ++s) w[s] = conv_w[c * AB_K1 + s];
#pragma unroll
  for (int s = 0; s < AB_K2; ++s) w[AB_K1 + s] = conv_w[AB_K1 * C + c * AB_K2 + s];
#pragma unroll
  for (int s = 0; s < AB_K3; ++s) w[AB_K1 + AB_K2 + s] = conv_w[(AB_K1 + AB_K2) * C + c * AB_K3 + s];
}

// partner exchange within rows of 16 lanes (DPP): lane i of a row reads lane i ^ 8
// (rotate by 8), 7 - i within each half row (half mirror), i ^ 2 and i ^ 1 (quad
// permutes)
__device__ __forceinline__ float dpp_ror8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_hmirror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));
}
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));
}

// Reduce-scatter of 26 values over the wave: returns, in lanes 2k and 2k + 1,
// the sum over the 64 lanes of v[k] (k < 26; lanes 52..63 return 0). Each level
// halves the values a lane holds and pairs it with a lane that holds the other
// half: lanes l and l + 32 (permlane32 swap), rows 2r and 2r + 1 (permlane16
// swap), then within rows by DPP; after the level on lane bit b the lane keeps
// the half selected by that bit, so value index k ends in lanes with l >> 1 = k.
__device__ __forceinline__ float ab_reduce_scatter(const float (&v)[AB_NV], int lane) {
  float a[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float y = k + 16 < AB_NV ? v[k + 16] : 0.f;
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(y), false, false);
    a[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // lanes < 32: value k; lanes >= 32: k + 16
  }
  float b[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a[k]), __float_as_uint(a[k + 8]), false, false);
    b[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);  // even rows: a index k; odd rows: k + 8
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) c[k] = (b3 ? b[k + 4] : b[k]) + dpp_ror8(b3 ? b[k] : b[k + 4]);
  float d[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) d[k] = (b2 ? c[k + 2] : c[k]) + dpp_hmirror(b2 ? c[k] : c[k + 2]);
  const float e = (b1 ? d[1] : d[0]) + dpp_xor2(b1 ? d[0] : d[1]);
  return e + dpp_xor1(e);
}

// CPT channels per thread (2: adjacent channel pairs, C even, rows aligned to a
// pair): the products of a thread's channels are added before the one
// reduce-scatter per token, so each cross-lane exchange serves 2x the channels.
template <typename TF, int CPT>
__device__ __forceinline__ void ab_ld_pair(const TF* row, uint32_t off, float (&v)[CPT]) {
  if constexpr (CPT == 1) {
    v[0] = ab_ldo(row, off);
  } else if constexpr (sizeof(TF) == 2) {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(row) + off);
    v[0] = __uint_as_float(u << 16);
    v[1] = __uint_as_float(u & 0xffff0000u);
  } else {
    const float2 u = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(row) + off);
    v[0] = u.x;
    v[1] = u.y;
  }
}

template <typename TF, int ST, int CPT>  // ST: tokens per strip; CPT: channels per thread
__global__ __launch_bounds__(256) void aug_bwd_gram_kernel(const TF* __restrict__ F, int64_t T, int64_t S, int64_t C,
                                                           const float* __restrict__ conv_w,
                                                           const float* __restrict__ dV, float* __restrict__ part) {
  __shared__ float red[2][AB_GRP][4][AB_NV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + tid) * CPT;
  const bool cok = c0 < C;  // lanes past C load zeros, so their products vanish (C % CPT == 0)
  const int64_t c = cok ? c0 : C - CPT;
  const int64_t t0 = (int64_t)blockIdx.y * ST;
  const int64_t t1 = t0 + ST < T ? t0 + ST : T;
  float w[CPT][AB_TAPS];
#pragma unroll
  for (int e = 0; e < CPT; ++e) ab_taps(conv_w, C, c + e, w[e]);
  const uint32_t ofF = (uint32_t)c * (uint32_t)sizeof(TF), ofV = (uint32_t)c * 4u;
  float win[CPT][12];  // before the first token: F_out[t0-12..t0-1] as loaded (rows < 0 masked at use)
#pragma unroll
  for (int s = 0; s < 12; ++s) {
    const int64_t tt = t0 - 12 + s;
    float x[CPT];
    ab_ld_pair<TF, CPT>(F + (tt >= 0 ? tt : 0) * C, ofF, x);  // loaded unconditionally, then selected
#pragma unroll
    for (int e = 0; e < CPT; ++e) win[e][s] = cok ? x[e] : 0.f;
  }
  struct Ld {
    float f[AB_PF][CPT], dv[AB_PF][4][CPT];
  };
  // CLAMP: rows past T read row T - 1 (the strip's last group)
  auto load = [&](int64_t tb, Ld& L, bool clamp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) {
      const int64_t t = clamp && tb + i >= T ? T - 1 : tb + i;
      float x[CPT];
      ab_ld_pair<TF, CPT>(F + t * C, ofF, x);  // loaded unconditionally, then selected
#pragma unroll
      for (int e = 0; e < CPT; ++e) L.f[i][e] = cok ? x[e] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[CPT];
        ab_ld_pair<float, CPT>(dV + (t * 4 + j) * C, ofV, y);
#pragma unroll
        for (int e = 0; e < CPT; ++e) L.dv[i][j][e] = cok ? y[e] : 0.f;
      }
    }
  };
  // one token: windows advanced by the rows `f`, products of the token's
  // components with dv summed over the thread's channels, their wave sums into
  // red[rb][gi]
  auto token = [&](const float (&f)[CPT], const float (&dv)[4][CPT], int64_t ts, bool masked, int rb, int gi)
                   __attribute__((always_inline)) {
    float v[AB_NV];
#pragma unroll
    for (int n = 0; n < AB_NV; ++n) v[n] = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
#pragma unroll
      for (int s = 0; s < 11; ++s) win[e][s] = win[e][s + 1];
      win[e][11] = f[e];
      float wm[12], u[4];
      if (masked) ab_mask(win[e], ts, wm);
      else
#pragma unroll
        for (int s = 0; s < 12; ++s) wm[s] = win[e][s];
      ab_convs(w[e], wm, u);
      int n = 0;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int k = a; k < 4; ++k) v[n++] += u[a] * u[k];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int a = 0; a < 4; ++a) v[10 + 4 * j + a] += dv[j][e] * u[a];
    }
    const float r = ab_reduce_scatter(v, lane);
    if (!(lane & 1) && (lane >> 1) < AB_NV) red[rb][gi][wave][lane >> 1] = r;
  };
  int64_t tb = t0, ts = t0 % S;  // ts: position of token tb in its sequence
  int rb = 0;                    // LDS buffer of the current 16-token group
  // after every 32 tokens and at the strip's end the waves' sums are added and stored
  auto flush = [&](int gi0, int64_t nb) __attribute__((always_inline)) {
    if (gi0 + AB_PF == AB_GRP || nb >= t1) {
      lds_barrier();
      const int64_t g0 = tb - gi0;
      const int ng = (int)(t1 - g0 < AB_GRP ? t1 - g0 : AB_GRP);  // tokens of the group inside the strip
#pragma unroll
      for (int e = tid; e < AB_NV * AB_GRP; e += 256) {
        const int k = e / AB_GRP, q = e & (AB_GRP - 1);
        if (q < ng) {
          const float* rr = &red[rb][q][0][k];
          part[((int64_t)blockIdx.x * AB_NV + k) * T + g0 + q] = ((rr[0] + rr[AB_NV]) + rr[2 * AB_NV]) + rr[3 * AB_NV];
        }
      }
      rb ^= 1;
    }
  };
  // one load group of AB_PF tokens tb.. while the next group loads. Fast: every
  // token inside the strip, at least 11 past its sequence start, and the next
  // group's rows inside T. General: tokens past t1 are computed on clamped rows
  // and never stored, and the window is masked per token.
  auto step_fast = [&](Ld& cur, Ld& nxt) __attribute__((always_inline)) {
    const int64_t nb = tb + AB_PF;
    load(nb, nxt, false);
    const int gi0 = (int)((tb - t0) & (AB_GRP - 1));
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) token(cur.f[i], cur.dv[i], 0, false, rb, gi0 + i);
    ts = ts + AB_PF == S ? 0 : ts + AB_PF;  // the pair's condition keeps ts + AB_PF <= S
    flush(gi0, nb);
    tb = nb;
  };
  auto step_general = [&](Ld& cur, Ld& nxt) __attribute__((always_inline)) {
    const int64_t nb = tb + AB_PF;
    load(nb, nxt, true);
    const int gi0 = (int)((tb - t0) & (AB_GRP - 1));
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) {
      token(cur.f[i], cur.dv[i], ts, true, rb, gi0 + i);
      ts = ts + 1 == S ? 0 : ts + 1;
    }
    flush(gi0, nb);
    tb = nb;
    return nb < t1;
  };
  Ld a, b;
  load(t0, a, true);
  for (;;) {  // pairs of groups keep the roles of a and b fixed
    while (tb + 3 * AB_PF <= T && tb + 2 * AB_PF <= t1 && ts >= 11 && ts + 2 * AB_PF <= S) {
      step_fast(a, b);
      step_fast(b, a);
    }
    if (tb >= t1 || !step_general(a, b) || !step_general(b, a)) break;
  }
}

// A workgroup of 256 threads takes 64 tokens: the channel groups' sums are
// added in order (float64) by all threads into LDS, then one thread per token
// forms P and Q in float64.
__global__ __launch_bounds__(256) void aug_bwd_coef_kernel(const float* __restrict__ part, int64_t T, int nq,
                                                           float* __restrict__ coef) {
  __shared__ double sd[AB_NV][64];
  const int tid = threadIdx.x;
  const int64_t tb = (int64_t)blockIdx.x * 64;
  for (int e = tid; e < AB_NV * 64; e += 256) {
    const int k = e >> 6, tl = e & 63;
    const int64_t tt = tb + tl < T ? tb + tl : T - 1;
    const float* pp = part + (int64_t)k * T + tt;
    const int64_t qs = (int64_t)AB_NV * T;
    double s = 0.0;
    int q = 0;
    for (; q + 8 <= nq; q += 8) {  // eight loads in flight, added in order
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = pp[(q + i) * qs];
#pragma unroll
      for (int i = 0; i < 8; ++i) s += (double)v[i];
    }
    for (; q < nq; ++q) s += (double)pp[q * qs];
    sd[k][tl] = s;
  }
  __syncthreads();
  const int64_t t = tb + tid;
  if (tid >= 64 || t >= T) return;
  double sv[AB_NV];
#pragma unroll
  for (int k = 0; k < AB_NV; ++k) sv[k] = sd[k][tid];
  double G[4][4], M[4][4];
  {
    int n = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = i; k < 4; ++k) G[i][k] = G[k][i] = sv[n++];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) M[j][i] = sv[10 + 4 * j + i];
  }
  auto gdot = [&](const double* a, const double* b) {  // <sum a_k u_k, sum b_l u_l>
    double r = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int l = 0; l < 4; ++l) r += a[k] * G[k][l] * b[l];
    return r;
  };
  // forward: V_j = sum_k B[j][k] u_k, with each step's n = <v, V_i>, d = <V_i, V_i>
  double B[4][4] = {{1, 0, 0, 0}, {0, 1, 0, 0}, {0, 0, 1, 0}, {0, 0, 0, 1}};
  double nn[4][4], dd[4][4];
#pragma unroll
  for (int j = 1; j < 4; ++j) {
    double v[4] = {0, 0, 0, 0};
    v[j] = 1.0;
#pragma unroll
    for (int i = 0; i < j; ++i) {
      const double n = gdot(v, B[i]), d = gdot(B[i], B[i]);
      nn[j][i] = n;
      dd[j][i] = d;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] -= (n / d) * B[i][k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) B[j][k] = v[k];
  }
  // reverse: a gradient vector is sum_q ga[q] dV_q + sum_k gb[k] u_k; the vector
  // before step (j, i) is recovered from the one after it: v_old = v + (n / d) V_i
  double ga[4][4] = {{1, 0, 0, 0}, {0, 1, 0, 0}, {0, 0, 1, 0}, {0, 0, 0, 1}}, gb[4][4] = {};
#pragma unroll
  for (int j = 3; j >= 1; --j) {
    double a[4], b[4], vo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      a[k] = ga[j][k];
      b[k] = gb[j][k];
      vo[k] = B[j][k];
    }
#pragma unroll
    for (int i = j - 1; i >= 0; --i) {
      const double n = nn[j][i], d = dd[j][i];
#pragma unroll
      for (int k = 0; k < 4; ++k) vo[k] += (n / d) * B[i][k];
      double p = 0.0;  // <V_i, g>
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        double gk = 0.0;  // <u_k, g>
#pragma unroll
        for (int q = 0; q < 4; ++q) gk += M[q][k] * a[q];
#pragma unroll
        for (int l = 0; l < 4; ++l) gk += G[k][l] * b[l];
        p += B[i][k] * gk;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ga[i][k] += -(n / d) * a[k];
        gb[i][k] += -(n / d) * b[k] - p * (vo[k] / d - 2.0 * n * B[i][k] / (d * d));
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] -= (p / d) * B[i][k];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      coef[t * 32 + j * 4 + k] = (float)a[k];
      coef[t * 32 + 16 + j * 4 + k] = (float)b[k];
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    coef[t * 32 + k] = (float)ga[0][k];
    coef[t * 32 + 16 + k] = (float)gb[0][k];
  }
}

template <typename TF, int ST>  // ST: tokens per strip
__global__ __launch_bounds__(256) void aug_bwd_walk_kernel(const TF* __restrict__ F, int64_t T, int64_t S, int64_t C,
                                                           const float* __restrict__ conv_w,
                                                           const float* __restrict__ dV,
                                                           const float* __restrict__ coef, TF* __restrict__ dF,
                                                           float* __restrict__ wpart) {
  __shared__ __attribute__((aligned(16))) float cfs[(ST + 11) * 32];
  const int tid = threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.x * 256 + tid;
  const bool cok = c0 < C;
  const int64_t c = cok ? c0 : C - 1;
  const int64_t t0 = (int64_t)blockIdx.y * ST;
  const int64_t t1 = t0 + ST < T ? t0 + ST : T;  // strip [t0, t1)
  // the walk starts up to 11 tokens after the strip, inside t1 - 1's sequence
  const int64_t se = (t1 - 1) - (t1 - 1) % S + S;  // end of that sequence
  const int64_t top = (t1 + 11 < se ? t1 + 11 : se) - 1;
  {  // P, Q of tokens t0..top into LDS
    const float4* src = reinterpret_cast<const float4*>(coef + t0 * 32);
    float4* dst = reinterpret_cast<float4*>(cfs);
    for (int64_t e = tid; e < (top - t0 + 1) * 8; e += 256) dst[e] = src[e];
  }
  float w[AB_TAPS];
  ab_taps(conv_w, C, c, w);
  float dw[AB_TAPS];
#pragma unroll
  for (int k = 0; k < AB_TAPS; ++k) dw[k] = 0.f;
  // acc[d]: what the tokens after t, within t's sequence, add to dF_out[t - d]
  // through the convs' transpose
  float acc[11];
#pragma unroll
  for (int d = 0; d < 11; ++d) acc[d] = 0.f;
  float win[12];  // F_out[t-11..t] as loaded (rows < 0 masked at use)
#pragma unroll
  for (int s = 0; s < 12; ++s) {
    const int64_t tt = top - 11 + s;
    win[s] = ab_ld(F + (tt >= 0 ? tt : 0) * C + c);
  }
  // load group of tokens tb, tb - 1, ..: F_out[t - 12] (the row entering the
  // window after t) and dV[t]
  struct Ld {
    float f[AB_PF], dv[AB_PF][4];
  };
  const uint32_t ofF = (uint32_t)c * (uint32_t)sizeof(TF), ofV = (uint32_t)c * 4u;
  // CLAMP: tokens below t0 read t0's rows, rows < 0 row 0 (masked at use)
  auto load = [&](int64_t tb, Ld& L, bool clamp) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) {
      const int64_t t = clamp && tb - i < t0 ? t0 : tb - i;
      L.f[i] = ab_ldo(F + (clamp && t < 12 ? 0 : t - 12) * C, ofF);
#pragma unroll
      for (int j = 0; j < 4; ++j) L.dv[i][j] = ab_ldo(dV + (t * 4 + j) * C, ofV);
    }
  };
  // one token t (ts: its position in the sequence). GENERAL: the window masked
  // at the sequence start, the transpose's sums cleared when t starts its
  // sequence, and dF_out and the tap sums taken only for t in [t0, t1) (the
  // group may hold halo tokens and, at the end, tokens below t0).
  auto token = [&](float fnext, const float (&dv)[4], int64_t t, int64_t ts, bool general)
                   __attribute__((always_inline)) {
    float wm[12], u[4];
    if (general) ab_mask(win, ts, wm);
    else
#pragma unroll
      for (int s = 0; s < 12; ++s) wm[s] = win[s];
    ab_convs(w, wm, u);
    const float4* cp = reinterpret_cast<const float4*>(cfs + (t - t0) * 32);
    float dU[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float4 pr = cp[r], qr = cp[4 + r];
      dU[r] = pr.x * dv[0] + pr.y * dv[1] + pr.z * dv[2] + pr.w * dv[3] + qr.x * u[0] + qr.y * u[1] + qr.z * u[2] +
              qr.w * u[3];
    }
    const float g = acc[0] + dU[0] + w[AB_K1 - 1] * dU[1] + w[AB_K1 + AB_K2 - 1] * dU[2] + w[AB_TAPS - 1] * dU[3];
    const bool in = !general || (t >= t0 && t < t1);
    if (in && cok) {
      char* row = reinterpret_cast<char*>(dF + t * C) + ofF;
      if constexpr (sizeof(TF) == 2) *reinterpret_cast<uint16_t*>(row) = (uint16_t)f2bf(g);
      else *reinterpret_cast<float*>(row) = g;
    }
    // dU_j[t] reaches dF_out[t - d] with tap w_j[kappa_j - 1 - d], d < kappa_j
#pragma unroll
    for (int d = 1; d < 12; ++d) {
      float a = d < 11 ? acc[d] : 0.f;
      if (d < AB_K1) a += w[AB_K1 - 1 - d] * dU[1];
      if (d < AB_K2) a += w[AB_K1 + AB_K2 - 1 - d] * dU[2];
      a += w[AB_TAPS - 1 - d] * dU[3];
      acc[d - 1] = general && ts == 0 ? 0.f : a;  // t - 1 lies in the previous sequence
    }
    float e1 = dU[1], e2 = dU[2], e3 = dU[3];
    if (general && !in) e1 = e2 = e3 = 0.f;
#pragma unroll
    for (int s = 0; s < AB_K1; ++s) dw[s] += e1 * wm[12 - AB_K1 + s];
#pragma unroll
    for (int s = 0; s < AB_K2; ++s) dw[AB_K1 + s] += e2 * wm[12 - AB_K2 + s];
#pragma unroll
    for (int s = 0; s < AB_K3; ++s) dw[AB_K1 + AB_K2 + s] += e3 * wm[12 - AB_K3 + s];
#pragma unroll
    for (int s = 11; s > 0; --s) win[s] = win[s - 1];
    win[0] = fnext;
  };
  __syncthreads();
  int64_t tb = top, ts = top % S;  // ts: position of token tb in its sequence
  // one load group of AB_PF tokens tb, tb - 1, .. while the next group loads.
  // Fast: every token inside the strip and at least 11 past its sequence start,
  // the next group's tokens not below t0. General: everything else.
  auto step_fast = [&](Ld& cur, Ld& nxt) __attribute__((always_inline)) {
    const int64_t nb = tb - AB_PF;
    load(nb, nxt, false);
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) token(cur.f[i], cur.dv[i], tb - i, 0, false);
    ts -= AB_PF;  // the pair's condition keeps ts >= AB_PF
    tb = nb;
  };
  auto step_general = [&](Ld& cur, Ld& nxt) __attribute__((always_inline)) {
    const int64_t nb = tb - AB_PF;
    load(nb, nxt, true);  // tokens below t0 clamped: the last group's loads go unused
#pragma unroll
    for (int i = 0; i < AB_PF; ++i) {
      token(cur.f[i], cur.dv[i], tb - i, ts, true);
      ts = ts == 0 ? S - 1 : ts - 1;
    }
    tb = nb;
    return nb >= t0;
  };
  Ld a, b;
  load(top, a, true);
  for (;;) {  // pairs of groups keep the roles of a and b fixed
    // (the pair's loads reach token tb - 3 AB_PF + 1 and its row tb - 3 AB_PF - 11)
    while (tb < t1 && tb - 3 * AB_PF + 1 >= t0 && tb >= 3 * AB_PF + 11 && ts >= 11 + 2 * AB_PF - 1) {
      step_fast(a, b);
      step_fast(b, a);
    }
    if (tb < t0 || !step_general(a, b) || !step_general(b, a)) break;
  }
  if (cok) {
#pragma unroll
    for (int k = 0; k < AB_TAPS; ++k) wpart[((int64_t)blockIdx.y * AB_TAPS + k) * C + c] = dw[k];
  }
}

// dconv_w in conv_w's layout from the strips' sums (strip order); one thread per
// (tap, channel).
__global__ __launch_bounds__(256) void aug_bwd_wsum_kernel(const float* __restrict__ wpart, int nstrip, int64_t C,
                                                           float* __restrict__ dconv) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= C * AB_TAPS) return;
  const int k = (int)(g / C);
  const int64_t c = g - k * C;
  float s = 0.f;
  for (int q = 0; q < nstrip; ++q) s += wpart[((int64_t)q * AB_TAPS + k) * C + c];
  int64_t o;
  if (k < AB_K1) o = c * AB_K1 + k;
  else if (k < AB_K1 + AB_K2) o = AB_K1 * C + c * AB_K2 + (k - AB_K1);
  else o = (AB_K1 + AB_K2) * C + c * AB_K3 + (k - AB_K1 - AB_K2);
  dconv[o] = s;
}

int ncu_of_device() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
    ncu = 256;
  return ncu;
}

int64_t al256(int64_t b) { return (b + 255) / 256 * 256; }

// token-tile groups of the dX pass (and of its dphi partials): about one
// workgroup per CU over the chunks and the nz stream groups (grid z), at most
// the tile count
int dx_groups(int64_t T, int64_t C, int nz) {
  const int64_t nchunk = (C + XCH - 1) / XCH * nz, ntile = (T + XT - 1) / XT;
  int64_t g = (int64_t)ncu_of_device() / nchunk;
  g = g < 1 ? 1 : g;
  return (int)(g < ntile ? g : ntile);
}

struct BwdWs {
  void* packed;
  float* partial;
  uint4* phi_rows;
  float *h_pre, *h_post, *h_res, *dP, *g2, *red, *dphi_part;
  int G;
};

// Workspace pieces in order, each 256-byte aligned, for a backward whose phi
// has nrows rows and ncol columns (packed B-operand form of pbytes, partials
// of qbytes); h_post [T, 4] only for the xHC route, h_pre [T, hp] otherwise.
BwdWs carve(void* ws, int64_t T, int64_t C, int64_t nrows, int ncol, int64_t pbytes, int64_t qbytes, int hp,
            bool route, int64_t* total) {
  BwdWs w{};
  unsigned char* p = (unsigned char*)ws;
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    unsigned char* q = p ? p + off : nullptr;
    off += al256(bytes);
    return q;
  };
  w.packed = take(pbytes);
  w.partial = (float*)take(qbytes);
  w.phi_rows = (uint4*)take(nrows * 128);
  w.h_pre = (float*)take(T * hp * 4);
  w.h_post = route ? (float*)take(T * 16 * 4) : nullptr;
  w.h_res = (float*)take(T * 16 * 4);
  w.dP = (float*)take(T * DPS * 4);
  w.g2 = (float*)take(T * 4);
  w.red = (float*)take((T + 15) / 16 * RED * 4);
  // dphi partials: one per group of the dX pass (pre: over the N / 4 stream groups)
  w.G = dx_groups(T, C, hp > 4 ? hp / 4 : 1);
  w.dphi_part = (float*)take((int64_t)w.G * nrows * ncol * 4);
  if (total) *total = off;
  return w;
}

BwdWs carve_mhc(void* ws, int64_t T, int64_t C, int64_t* total) {
  return carve(ws, T, C, BS * C, BCOL, fast_bwd_packed_bytes(C), fast_bwd_partial_bytes(T, C), 4, false, total);
}
// route with K components: phi_act [4C, 4K + 16] packed as NB = 4 blocks of 16
// columns, 2 hi and 2 lo (2 x 8 NB 16-byte chunks per 8 rows)
BwdWs carve_route(void* ws, int64_t T, int64_t C, int K, int64_t* total) {
  const int nb = 4;
  return carve(ws, T, C, BS * C, 4 * K + 16, BS * C / 8 * (16 * nb) * 16, fast_xroute_partial_bytes(T, C, K), 4,
               true, total);
}
// pre: phi_pre [NC, N] packed as 2 x 16 columns
BwdWs carve_pre(void* ws, int64_t T, int N, int64_t C, int64_t* total) {
  return carve(ws, T, C, (int64_t)N * C, N, (int64_t)N * C / 8 * 32 * 16, fast_xpre_partial_bytes(T, N, C), N, false,
               total);
}

hipError_t launch_sums(const BwdWs& w, int64_t T, int64_t nrows, int ncol, float* dphi, float* dbias, int na0,
                       int na, float* dalpha, hipStream_t st) {
  const int64_t nphi = nrows * ncol, nbp = (nphi + 255) / 256;
  hipLaunchKernelGGL(bwd_sums_kernel, dim3((unsigned)(nbp + ncol + na)), dim3(256), 0, st, w.dphi_part, nphi, w.G,
                     (int)nbp, dphi, w.red, (T + 15) / 16, ncol, dbias, na0, dalpha);
  return hipGetLastError();
}

}  // namespace

bool fast_backward_supported(int dtype, int n, int64_t T, int64_t C, int iters) {
  return dtype == 1 && n == 4 && T >= 1 && iters >= 1 && iters <= HC_MAX_BWD_ITERS && C % 32 == 0 && C >= 32 &&
         fast_coeffs_partial_bytes(T, 4, C, 1) > 0 && (C + FCH - 1) / FCH <= 65535 &&
         (int64_t)XT * 4 * C * 2 < (1ll << 32);  // a dX tile's rows in one buffer resource
}

int64_t fast_backward_ws_bytes(int64_t T, int64_t C) {
  int64_t total = 0;
  carve_mhc(nullptr, T, C, &total);
  return total;
}

hipError_t launch_fast_backward_post(const void* X, int64_t T, int64_t C, const float* h_post, const void* F_out,
                                     const void* dX_next, void* dF_out, float* dh, hipStream_t st) {
  hipLaunchKernelGGL((bwd_post_kernel<BM_MHC, 1>), dim3((unsigned)T), dim3(256), 0, st, (const uint16_t*)X,
                     (const uint16_t*)dX_next, (const uint16_t*)F_out, C, 4, (const int32_t*)nullptr, h_post, dh,
                     BCOL, 4, dF_out);
  return hipGetLastError();
}

hipError_t launch_fast_backward(const void* X, int64_t T, int64_t C, const float* phi, const float* bias,
                                float a_pre, float a_post, float a_res, int iters, const void* dX_next,
                                const void* dF_in, float* dh, void* dX, float* dphi, float* dbias, float* dalpha,
                                void* ws, hipStream_t st) {
  const BwdWs w = carve_mhc(ws, T, C, nullptr);
  const uint16_t* x = (const uint16_t*)X;
  // the projection recompute also forms dH_pre from the same read of x
  hipError_t e = launch_fast_bwd_front(X, T, C, phi, w.packed, w.phi_rows, w.partial, dF_in, st);
  if (e != hipSuccess) return e;
  if ((e = launch_fast_bwd_coeffs(w.partial, T, C, bias, a_pre, a_post, a_res, iters, dh, w.dP, w.g2, w.red,
                                  w.h_pre, w.h_res, st)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(bwd_dx_kernel<BM_MHC>, dim3((unsigned)((C + XCH - 1) / XCH), (unsigned)w.G), dim3(512), 0, st,
                     x, (const uint16_t*)dX_next, (const uint16_t*)dF_in, T, C, 4, (const int32_t*)nullptr, w.h_pre,
                     w.h_res, w.dP, w.g2, w.phi_rows, (uint16_t*)dX, BCOL, (int64_t)BS * C, w.dphi_part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_sums(w, T, (int64_t)BS * C, BCOL, dphi, dbias, 32, 3, dalpha, st);
}

// ------------------------------------------------------------------ xHC

bool fast_xhc_backward_supported(int dtype, int N, int k, int K, int64_t T, int64_t C, int iters) {
  return dtype == 1 && N % 4 == 0 && N >= 4 && N <= 16 && k == 4 && (K == 1 || K == 4) && T >= 1 && iters >= 1 &&
         iters <= HC_MAX_BWD_ITERS && C % 32 == 0 && C >= 32 && C < (1ll << 24) &&
         // the projection partials are addressed with 32-bit buffer offsets
         fast_xroute_partial_bytes(T, C, K) < (1ll << 31) && fast_xpre_partial_bytes(T, N, C) < (1ll << 31) &&
         (C + FCH - 1) / FCH <= 65535 && T * (int64_t)N * C < (1ll << 40) &&
         (int64_t)XT * N * C * 2 < (1ll << 32);  // a dX tile's rows in one buffer resource
}

int64_t fast_xhc_backward_ws_bytes(int64_t T, int N, int64_t C) {
  int64_t a = 0, b = 0, c = 0;
  carve_route(nullptr, T, C, 1, &a);
  carve_route(nullptr, T, C, 4, &c);
  carve_pre(nullptr, T, N, C, &b);
  a = a > c ? a : c;
  return a > b ? a : b;
}

hipError_t launch_fast_xroute_backward(const void* X, int64_t T, int N, int64_t C, const int32_t* idx,
                                       const float* phi_act, const float* b_act, float a_post, float a_res, int iters,
                                       const void* Wb, int K, void* dX, void* dWb, float* dphi_act, float* db_act,
                                       float* dalpha, float* dh, void* ws, hipStream_t st) {
  const BwdWs w = carve_route(ws, T, C, K, nullptr);
  const uint16_t* x = (const uint16_t*)X;
  const int ncol = 4 * K + 16;
  // the active set's maps (the forward's kernels) and its projection partials
  hipError_t e = launch_fast_xhc_active(X, T, N, C, idx, K, phi_act, b_act, a_post, a_res, iters, w.h_post, w.h_res,
                                        w.packed, w.partial, st, w.phi_rows);
  if (e != hipSuccess) return e;
  if (K == 4)
    hipLaunchKernelGGL((bwd_post_kernel<BM_ROUTE, 4>), dim3((unsigned)T), dim3(256), 0, st, x, (const uint16_t*)dX,
                       (const uint16_t*)Wb, C, N, idx, w.h_post, dh, ncol, 0, dWb);
  else
    hipLaunchKernelGGL((bwd_post_kernel<BM_ROUTE, 1>), dim3((unsigned)T), dim3(256), 0, st, x, (const uint16_t*)dX,
                       (const uint16_t*)Wb, C, N, idx, w.h_post, dh, ncol, 0, dWb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_fast_xroute_bwd_coeffs(w.partial, T, C, K, b_act, a_post, a_res, iters, dh, w.dP, w.g2, w.red,
                                         w.h_res, st)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(bwd_dx_kernel<BM_ROUTE>, dim3((unsigned)((C + XCH - 1) / XCH), (unsigned)w.G), dim3(512), 0, st,
                     x, (const uint16_t*)dX, (const uint16_t*)nullptr, T, C, N, idx, (const float*)nullptr, w.h_res,
                     w.dP, w.g2, w.phi_rows, (uint16_t*)dX, ncol, (int64_t)BS * C, w.dphi_part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dalpha: the post and res gate sums (red columns 33, 34)
  return launch_sums(w, T, (int64_t)BS * C, ncol, dphi_act, db_act, 33, 2, dalpha, st);
}

hipError_t launch_fast_xpre_backward(const void* X, int64_t T, int N, int64_t C, const float* phi_pre,
                                     const float* b_pre, float a_pre, const void* dF_in, void* dX, float* dphi_pre,
                                     float* db_pre, float* dalpha, float* dh_pre, void* ws, hipStream_t st) {
  const BwdWs w = carve_pre(ws, T, N, C, nullptr);
  const uint16_t* x = (const uint16_t*)X;
  // the projection recompute also forms dH_pre = <dF_in, x_i> (same read of the state)
  hipError_t e = launch_fast_xpre_bwd_front(X, T, N, C, phi_pre, dF_in, w.packed, w.phi_rows, w.partial, st);
  if (e != hipSuccess) return e;
  if ((e = launch_fast_xpre_bwd_coeffs(w.partial, T, N, C, b_pre, a_pre, dh_pre, w.dP, w.g2, w.red, w.h_pre, st)) !=
      hipSuccess)
    return e;
  const unsigned ng = (unsigned)(N / 4);
  hipLaunchKernelGGL(bwd_dx_kernel<BM_PRE>, dim3((unsigned)((C + XCH - 1) / XCH), (unsigned)w.G, ng), dim3(512), 0,
                     st, x, (const uint16_t*)dX, (const uint16_t*)dF_in, T, C, N, (const int32_t*)nullptr, w.h_pre,
                     (const float*)nullptr, w.dP, w.g2, w.phi_rows, (uint16_t*)dX, N, (int64_t)N * C, w.dphi_part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dalpha: the gate sum (red column 32)
  return launch_sums(w, T, (int64_t)N * C, N, dphi_pre, db_pre, 32, 1, dalpha, st);
}


// --------------------------------------------- augmentation backward (host)

bool fast_augment_backward_supported(int dtype, int64_t B, int64_t S, int64_t C, const int* kappa, int r) {
  return (dtype == 0 || dtype == 1) && B >= 1 && S >= 1 && C >= 1 && r == 3 && kappa && kappa[0] == AB_K1 &&
         kappa[1] == AB_K2 && kappa[2] == AB_K3 && B * S * C < (1ll << 40);
}

// tokens per strip of the reverse walk: the longer strip (fewer halo tokens
// walked twice) while it leaves at least two workgroups per CU (walk at B = 2,
// S = 4096, C = 4096: 143 against 161 us)
int64_t aug_strip(int64_t T, int64_t C) {
  const int64_t nq = (C + 255) / 256;
  return nq * ((T + AB_STRIP2 - 1) / AB_STRIP2) >= 2 * (int64_t)ncu_of_device() ? AB_STRIP2 : AB_STRIP;
}

int64_t fast_augment_backward_ws_bytes(int64_t B, int64_t S, int64_t C) {
  // the tap partials are sized for the shorter strip (the most strips)
  const int64_t T = B * S, nq = (C + 255) / 256, nstrip = (T + AB_STRIP - 1) / AB_STRIP;
  return al256(nq * AB_NV * T * 4) + al256(T * 32 * 4) + al256(nstrip * AB_TAPS * C * 4);
}

hipError_t launch_fast_augment_backward(const void* F_out, int dtype, int64_t B, int64_t S, int64_t C,
                                        const float* conv_w, const float* dV, void* dF_out, float* dconv_w, void* ws,
                                        hipStream_t st) {
  const int64_t T = B * S, nq = (C + 255) / 256, strip = aug_strip(T, C), nstrip = (T + strip - 1) / strip;
  unsigned char* p = (unsigned char*)ws;
  float* part = (float*)p;
  float* coef = (float*)(p + al256(nq * AB_NV * T * 4));
  float* wpart = (float*)(p + al256(nq * AB_NV * T * 4) + al256(T * 32 * 4));
  const dim3 grid((unsigned)nq, (unsigned)nstrip), blk(256);
  // the Gram pass walks no halo: it keeps the shorter strips (more workgroups);
  // channel pairs per thread when C is even and the rows are pair-aligned
  const size_t fes = dtype == 1 ? 2 : 4;
  const bool pairs = C % 2 == 0 && reinterpret_cast<uintptr_t>(F_out) % (2 * fes) == 0 &&
                     reinterpret_cast<uintptr_t>(dV) % 8 == 0;
  const int64_t nqg = pairs ? (C + 511) / 512 : nq;  // channel groups of the Gram pass
  const dim3 ggrid((unsigned)nqg, (unsigned)((T + AB_STRIP - 1) / AB_STRIP));
#define HC_AUG_GRAM(TF, CPT)                                                                                       \
  hipLaunchKernelGGL((aug_bwd_gram_kernel<TF, AB_STRIP, CPT>), ggrid, blk, 0, st, (const TF*)F_out, T, S, C, conv_w, \
                     dV, part)
  if (dtype == 1) {
    if (pairs) HC_AUG_GRAM(uint16_t, 2);
    else HC_AUG_GRAM(uint16_t, 1);
  } else {
    if (pairs) HC_AUG_GRAM(float, 2);
    else HC_AUG_GRAM(float, 1);
  }
#undef HC_AUG_GRAM
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aug_bwd_coef_kernel, dim3((unsigned)((T + 63) / 64)), dim3(256), 0, st, part, T, (int)nqg, coef);
  if ((e = hipGetLastError()) != hipSuccess) return e;
#define HC_AUG_WALK(TF, ST)                                                                                 \
  hipLaunchKernelGGL((aug_bwd_walk_kernel<TF, ST>), grid, blk, 0, st, (const TF*)F_out, T, S, C, conv_w, dV, coef, \
                     (TF*)dF_out, wpart)
  if (dtype == 1) {
    if (strip == AB_STRIP2) HC_AUG_WALK(uint16_t, AB_STRIP2);
    else HC_AUG_WALK(uint16_t, AB_STRIP);
  } else {
    if (strip == AB_STRIP2) HC_AUG_WALK(float, AB_STRIP2);
    else HC_AUG_WALK(float, AB_STRIP);
  }
#undef HC_AUG_WALK
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(aug_bwd_wsum_kernel, dim3((unsigned)((C * AB_TAPS + 255) / 256)), dim3(256), 0, st, wpart,
                     (int)nstrip, C, dconv_w);
  return hipGetLastError();
}

}  // namespace hc
