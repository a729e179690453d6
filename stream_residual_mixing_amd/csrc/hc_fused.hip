// Fast paths for n = 4 bfloat16 streams on gfx950.
//
// mhc_stream_kernel<POST, PROJ> walks a tile of 16 tokens through all C
// channels of their 4 streams in 256-channel super-chunks:
//   POST: X_next = h_res X + h_post^T F_out  (mHC notes Eq. 3, F_post,res of 4.3.1)
//   PROJ: the skinny projection of the tile it streams (the X_next it just
//         produced when POST, else X) with MFMA, the sum of squares, and the
//         coefficient epilogue (Eq. 15-19): RMS factor, gates, sigmoid,
//         2*sigmoid and Sinkhorn-Knopp.
// The projection uses v_mfma_f32_16x16x32_bf16 with the tile's 16 tokens as
// the M rows. phi (float32) is split as phi = hi + lo with hi = bf16(phi) and
// lo = bf16(phi - hi), so X (exact in bf16) times hi plus X times lo carries
// about 16 significant bits of phi into an fp32 accumulator. phi is packed once
// per call into the B-operand order [row/8][48][8] (hi columns 0..23, lo
// columns 24..47), so each lane's 8 k-values of one column are 16 contiguous
// bytes.
#include <type_traits>

#include "hc_device.h"
#include "hc_fast.h"

namespace hc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int NS4 = 4;              // streams
constexpr int NCOL = 24;            // n*n + 2n
constexpr int NCP = 48;             // packed hi|lo columns
constexpr int TOK = 16;             // tokens per tile (MFMA M)

// ------------------------------------------------------------- phi packing

__global__ __launch_bounds__(256) void pack_phi_kernel(const float* __restrict__ phi, int64_t K,
                                                       uint16_t* __restrict__ packed) {
  // one thread per (row group of 8, column): writes the hi chunk (column c) and
  // the lo chunk (column NCOL + c), 8 bf16 each
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ngroups = K / 8;
  if (g >= ngroups * NCOL) return;
  const int64_t rg = g / NCOL;
  const int c = (int)(g - rg * NCOL);
  float p[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) p[e] = phi[(rg * 8 + e) * NCOL + c];
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const uint32_t h0 = f2bf(p[e]), h1 = f2bf(p[e + 1]);
    hi[e / 2] = h0 | (h1 << 16);
    // p - hi is exact in float32
    lo[e / 2] = f2bf(p[e] - bf2f(h0)) | (f2bf(p[e + 1] - bf2f(h1)) << 16);
  }
  uint4* out = reinterpret_cast<uint4*>(packed) + rg * NCP;
  out[c] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  out[NCOL + c] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
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
// = 8 waves) per 256-channel super-chunk of all 4 streams:
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

// Round-to-nearest-even pack of two floats into bf16x2 (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf2_hw(float a, float b) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  const b2_t r = __builtin_convertvector((f2_t){a, b}, b2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// v if keep, else zeros: per-component selects (a select between two uint4
// objects can become a select of their addresses, which puts them in scratch).
__device__ __forceinline__ uint4 keep_or_zero(bool keep, const uint4& v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// Cross-wave reduction of a 32-token tile and the coefficient epilogue
// ([mHC] Eq. 15-19). acc[tb][b] holds this wave's partial D = A * B for token
// block tb and packed column block b (lane: D[m = q*4 + e][n = tau]); gram[tb]
// holds its partial A * A^T, whose diagonal is the sum of squares. `red` is LDS
// scratch of at least SWAVE * TILE * (NCP + 1) + TILE * (NCOL + SWAVE + 1)
// floats; the caller has synchronised the workgroup before the call.
__device__ __forceinline__ void tile_epilogue(float* red, const floatx4_t (&acc)[2][3], const floatx4_t (&gram)[2],
                                              int64_t t0, int64_t T, int64_t C, const float* __restrict__ bias,
                                              Gate gate, int iters, float* __restrict__ h_pre_out,
                                              float* __restrict__ h_post_out, float* __restrict__ h_res_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tau = lane & 15, q = lane >> 4;
  float* Pt = red + SWAVE * TILE * (NCP + 1);   // [TILE][NCOL]
  float* ssr = Pt + TILE * NCOL;                // [SWAVE][TILE]
  float* sst = ssr + SWAVE * TILE;              // [TILE]
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int b = 0; b < 3; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(wave * TILE + tb * TOK + q * 4 + e) * (NCP + 1) + b * 16 + tau] = acc[tb][b][e];
  // the diagonal m == n of gram[tb] sits in the lane with tau == q*4 + e
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (tau == q * 4 + e) ssr[wave * TILE + tb * TOK + tau] = gram[tb][e];
  __syncthreads();
  for (int k = tid; k < TILE * NCOL; k += STHR) {
    const int m = k / NCOL, col = k - m * NCOL;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < SWAVE; ++w)
      sum += red[(w * TILE + m) * (NCP + 1) + col] + red[(w * TILE + m) * (NCP + 1) + NCOL + col];
    Pt[m * NCOL + col] = sum;
  }
  if (tid < TILE) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < SWAVE; ++w) sum += ssr[w * TILE + tid];
    sst[tid] = sum;
  }
  __syncthreads();
  // thread (token m, entry e) for 32 tokens x 16 entries
  const int m = tid >> 4, e = tid & 15;
  const int64_t tt = t0 + m;
  const float r = sqrtf(sst[m] / (float)(NS4 * C));
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  if (e < 8 && tt < T) {
    const float a = e < 4 ? gate.a_pre : gate.a_post;
    const float z = a * (Pt[m * NCOL + e] * invr) + bias[e];
    if (e < 4) {
      if (h_pre_out) h_pre_out[tt * 4 + e] = sigmoid(z);
    } else {
      h_post_out[tt * 4 + (e - 4)] = 2.0f * sigmoid(z);
    }
  }
  // h_res: Sinkhorn on the 4x4 block held by 16 consecutive lanes (i = e>>2, j = e&3)
  const float z = gate.a_res * (Pt[m * NCOL + 8 + e] * invr) + bias[8 + e];
  float zm = z;
  zm = fmaxf(zm, __shfl_xor(zm, 1, 64));
  zm = fmaxf(zm, __shfl_xor(zm, 2, 64));
  zm = fmaxf(zm, __shfl_xor(zm, 4, 64));
  zm = fmaxf(zm, __shfl_xor(zm, 8, 64));
  float M = expf(z - zm);
  for (int it = 0; it < iters; ++it) {
    float cs = M + __shfl_xor(M, 4, 64);  // column sum over i
    cs += __shfl_xor(cs, 8, 64);
    M = M / cs;
    float rs = M + __shfl_xor(M, 1, 64);  // row sum over j
    rs += __shfl_xor(rs, 2, 64);
    M = M / rs;
  }
  if (tt < T) h_res_out[tt * 16 + e] = M;
}

// Buffer resource over [base, base + bytes): stores whose offset falls outside are
// dropped by the hardware, so a guarded store needs no branch (a store behind a
// branch makes the compiler's wait counts conservative at the merge).
constexpr unsigned BUF_DW3 = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;  // any offset >= the range is dropped

template <bool POST, bool PROJ>
__global__ __launch_bounds__(STHR) void mhc_stream_kernel(
    const uint16_t* X, int64_t T, int64_t C,
    const float* __restrict__ h_res_in, const float* __restrict__ h_post_in,
    const uint16_t* __restrict__ F, uint16_t* Y,
    const uint16_t* __restrict__ phi_p, const float* __restrict__ bias, Gate gate, int iters,
    float* __restrict__ h_pre_out, float* __restrict__ h_post_out, float* __restrict__ h_res_out) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[PROJ ? 2 * LBUF : 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * TILE;
  // streaming-phase role: tokens st_tok and st_tok + 16 of the tile
  const int st_tok = tid >> 5;
  const int st_c8 = (tid & 31) * 8;
  int64_t st_t[2];
  bool st_ok[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    st_t[p] = t0 + st_tok + 16 * p;
    st_ok[p] = st_t[p] < T;
  }
  // MFMA-phase role
  const int tau = lane & 15;
  const int q = lane >> 4;
  const int64_t nsc = (C + SC - 1) / SC;


  // per-token post coefficients of the tile, in LDS: [TILE][20] = h_res (16) | h_post (4)
  __shared__ float coef[POST ? TILE * 20 : 1];
  if (POST) {
    for (int k = tid; k < TILE * 20; k += STHR) {
      const int m = k / 20, e = k - m * 20;
      const int64_t tt = t0 + m;
      coef[k] = tt < T ? (e < 16 ? h_res_in[tt * 16 + e] : h_post_in[tt * 4 + (e - 16)]) : 0.f;
    }
    __syncthreads();
  }
  floatx4_t acc[2][3], gram[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    gram[tb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 3; ++b) acc[tb][b] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Loads are unconditional: rows past T and channels past C are clamped to a
  // valid address and their values replaced by zeros, so no load sits behind a
  // branch and consecutive loads stay in flight together.
  // X_next of this tile through a buffer resource (rows t0 .. min(T, t0 + TILE))
  const int64_t nrow = (T - t0) < TILE ? (T - t0) : TILE;
  const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(
      POST ? Y + t0 * (NS4 * C) : nullptr, 0, POST ? (uint32_t)(nrow * NS4 * C * 2) : 0u, BUF_DW3);
  const uint16_t* xrow[2];
  const uint16_t* frow[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int64_t tc = st_ok[p] ? st_t[p] : T - 1;
    xrow[p] = X + tc * (NS4 * C);
    frow[p] = POST ? F + tc * C : nullptr;
  }

  // Loads of one token half (p = 0: tokens 0..15, p = 1: tokens 16..31 of the
  // tile) of super-chunk s.
  auto load_half = [&](int64_t s, auto P, uint4 (&xv)[NS4], uint4& fv) __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int64_t c = s * SC + st_c8;
    const int64_t cc = c < C ? c : C - 8;
#pragma unroll
    for (int i = 0; i < NS4; ++i) xv[i] = *reinterpret_cast<const uint4*>(xrow[p] + i * C + cc);
    if (POST) fv = *reinterpret_cast<const uint4*>(frow[p] + cc);
  };

  // Streaming work of one token half: X_next (POST), its squared norm and its
  // bf16 tile in LDS (PROJ).
  auto stream_half = [&](int64_t s, auto P, const uint4 (&xc)[NS4], const uint4& fc, unsigned char* buf)
                         __attribute__((always_inline)) {
    constexpr int p = decltype(P)::value;
    const int64_t c = s * SC + st_c8;
    const bool ok = st_ok[p] && c < C;
    const int m = st_tok + 16 * p;
    uint4 a_frag[NS4];
    if (POST) {
      const float* cf = coef + m * 20;
      float fv[8];
      unpack8(fc, fv);
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        float y[8];
        const float wp = cf[16 + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = wp * fv[e];
#pragma unroll
        for (int j = 0; j < NS4; ++j) {
          float xv[8];
          unpack8(xc[j], xv);
          const float w = cf[i * 4 + j];
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
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{o.x, o.y, o.z, o.w}, yres, yoff, 0, 2 /* nt */);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NS4; ++i) a_frag[i] = keep_or_zero(ok, xc[i]);
    }
    if (PROJ) {
#pragma unroll
      for (int i = 0; i < NS4; ++i) *reinterpret_cast<uint4*>(buf + (i * TILE + m) * LROW + st_c8 * 2) = a_frag[i];
    }
  };

  // One super-chunk. Issue order: B fragments of its MFMA phase, the second
  // token half of this super-chunk, then (after the first half is computed) the
  // first half of the next super-chunk. Waiting for the first half or for the
  // B fragments thus never waits for loads issued later; the first-half
  // register set is refilled for the next super-chunk while the second half
  // is computed. prefetch: Pre (load the next super-chunk's first half) or NoPre.
  uint4 xA[NS4], xB[NS4], fA = make_uint4(0, 0, 0, 0), fB = make_uint4(0, 0, 0, 0);
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  auto body = [&](int64_t s, auto prefetch) __attribute__((always_inline)) {
    const int64_t cg = s * SC + wave * 32;
    uint4 pf[NS4][3];
    if (PROJ) {
      const int64_t cgc = cg < C ? cg : C - 32;
#pragma unroll
      for (int i = 0; i < NS4; ++i) {
        const uint4* pb = reinterpret_cast<const uint4*>(phi_p) + ((i * C + cgc) / 8 + q) * NCP + tau;
#pragma unroll
        for (int b = 0; b < 3; ++b) pf[i][b] = pb[b * 16];
      }
    }
    load_half(s, H1{}, xB, fB);
    unsigned char* buf = lds + (s & 1) * LBUF;
    stream_half(s, H0{}, xA, fA, buf);
    if constexpr (decltype(prefetch)::value) load_half(s + 1, H0{}, xA, fA);
    stream_half(s, H1{}, xB, fB, buf);
    if (PROJ) {
      __syncthreads();
      // With POST, rows past T and channels past C hold values computed from
      // clamped loads (zeroing them before the store would turn the store into
      // a branch): their A fragments are replaced by zeros here. Without POST
      // the tile already holds zeros there. Either way a group past C adds
      // nothing against its clamped, valid B address.
      const bool ch_ok = cg + q * 8 < C;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const bool a_ok = ch_ok && (t0 + tb * TOK + tau < T);
#pragma unroll
        for (int i = 0; i < NS4; ++i) {
          uint4 af =
              *reinterpret_cast<const uint4*>(buf + (i * TILE + tb * TOK + tau) * LROW + (wave * 32 + q * 8) * 2);
          if (POST) af = keep_or_zero(a_ok, af);
#pragma unroll
          for (int b = 0; b < 3; ++b)
            acc[tb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(pf[i][b]), acc[tb][b], 0, 0, 0);
          // A times its own transpose: the diagonal accumulates each token's sum of squares.
          gram[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af), as_bf16x8(af), gram[tb], 0, 0, 0);
        }
      }
      // The next super-chunk writes the other buffer; the one after it writes this
      // buffer only after passing the next barrier, i.e. after these reads.
    }
  };

  // The last super-chunk has nothing to prefetch; it is peeled so that the
  // loop's prefetch is unconditional (branch-free wait counts).
  load_half(0, H0{}, xA, fA);
  for (int64_t s = 0; s + 1 < nsc; ++s) body(s, std::true_type{});
  body(nsc - 1, std::false_type{});
  if (!PROJ) return;

  __syncthreads();
  tile_epilogue(reinterpret_cast<float*>(lds), acc, gram, t0, T, C, bias, gate, iters, h_pre_out, h_post_out,
                h_res_out);
}

// --------------------------------------------------------------- pre-read

// F_in[t, c] = sum_i h_pre[t, i] X[t, i, c] for n = 4 bf16; 16 channels per thread.
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
  unpack8(*reinterpret_cast<const uint4*>(p), a);
  unpack8(*reinterpret_cast<const uint4*>(p + C), b);
  unpack8(*reinterpret_cast<const uint4*>(p + 2 * C), c);
  unpack8(*reinterpret_cast<const uint4*>(p + 3 * C), d);
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = w0 * a[e] + w1 * b[e] + w2 * c[e] + w3 * d[e];
  uint4 q;
  q.x = pack_bf2(o[0], o[1]);
  q.y = pack_bf2(o[2], o[3]);
  q.z = pack_bf2(o[4], o[5]);
  q.w = pack_bf2(o[6], o[7]);
  *reinterpret_cast<uint4*>(F_in + t * C + c0) = q;
}

// ----------------------------------------------------------------- hosts

static inline bool a16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int64_t fast_coeffs_packed_bytes(int n, int64_t C, int dtype) {
  if (n != 4 || dtype != 1 || C % 32 != 0) return 0;
  return (int64_t)n * C / 8 * NCP * 16;
}

bool fast_coeffs_supported(int dtype, int n, int64_t C, const void* X) {
  return dtype == 1 && n == 4 && C % 32 == 0 && C >= 32 && a16(X);
}

bool fast_post_supported(int dtype, int n, int64_t C, const void* X, const void* F, const void* Y) {
  return dtype == 1 && n == 4 && C % 32 == 0 && C >= 32 && a16(X) && a16(F) && a16(Y);
}

static hipError_t launch_pack(const float* phi, int64_t K, void* packed, hipStream_t st) {
  const int64_t work = K / 8 * NCOL;
  hipLaunchKernelGGL(pack_phi_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st, phi, K,
                     (uint16_t*)packed);
  return hipGetLastError();
}

hipError_t launch_fast_coeffs_pre(const void* X, int64_t T, int64_t C, const float* phi,
                                  const float* bias, float a_pre, float a_post, float a_res,
                                  int iters, float* h_pre, float* h_post, float* h_res, void* F_in,
                                  void* packed, float* h_pre_tmp, hipStream_t st) {
  hipError_t e = launch_pack(phi, 4 * C, packed, st);
  if (e != hipSuccess) return e;
  float* hp = h_pre ? h_pre : h_pre_tmp;
  const unsigned grid = (unsigned)((T + TILE - 1) / TILE);
  hipLaunchKernelGGL((mhc_stream_kernel<false, true>), dim3(grid), dim3(STHR), 0, st, (const uint16_t*)X, T, C,
                     nullptr, nullptr, nullptr, nullptr, (const uint16_t*)packed, bias,
                     Gate{a_pre, a_post, a_res}, iters, hp, h_post, h_res);
  e = hipGetLastError();
  if (e != hipSuccess || !F_in) return e;
  const int64_t work = T * (C / 8);
  hipLaunchKernelGGL(pre4_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st, (const uint16_t*)X, T,
                     C, hp, (uint16_t*)F_in);
  return hipGetLastError();
}

hipError_t launch_fast_pre(const void* X, int64_t T, int64_t C, const float* h_pre, void* F_in, hipStream_t st) {
  const int64_t work = T * (C / 8);
  hipLaunchKernelGGL(pre4_kernel, dim3((unsigned)((work + 255) / 256)), dim3(256), 0, st, (const uint16_t*)X, T,
                     C, h_pre, (uint16_t*)F_in);
  return hipGetLastError();
}

hipError_t launch_fast_post_coeffs(const void* X, int64_t T, int64_t C, const float* h_res,
                                   const float* h_post, const void* F, void* Y, const float* phi,
                                   const float* bias, float a_pre, float a_post, float a_res, int iters,
                                   float* h_pre_n, float* h_post_n, float* h_res_n, void* packed,
                                   hipStream_t st) {
  hipError_t e = launch_pack(phi, 4 * C, packed, st);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((T + TILE - 1) / TILE);
  hipLaunchKernelGGL((mhc_stream_kernel<true, true>), dim3(grid), dim3(STHR), 0, st, (const uint16_t*)X, T, C,
                     h_res, h_post, (const uint16_t*)F, (uint16_t*)Y, (const uint16_t*)packed, bias,
                     Gate{a_pre, a_post, a_res}, iters, h_pre_n, h_post_n, h_res_n);
  return hipGetLastError();
}

}  // namespace hc
