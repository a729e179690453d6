// Generic gfx950 kernels of libhc: any n, N, k, K, C and both stream dtypes.
//
// These kernels favour plain structure over speed: the projection runs on the
// vector ALUs with one workgroup per (token, 32-column chunk) and reads phi
// through the caches (or, when phi fits, from an LDS copy per workgroup), the
// coefficient epilogue uses one workgroup per token (16 lanes for 4 x 4
// residual maps), and the streaming kernels give each thread 8 consecutive
// channels of one token. The specialised fast paths (hc_fused.hip) cover the
// shapes that matter for throughput; everything else runs here.
#include "hc_device.h"
#include "hc_launch.h"

namespace hc {

// --------------------------------------------------------------------------
// Skinny projection P[t, :] = vec(x_t) @ [phiA | phiB] and ss[t] = ||vec x_t||^2
// (mHC notes Eq. 14-15; xHC summary: router and maps from the state).
// vec(x_t) is the concatenation of `nvec` stream rows of token t: rows 0..nvec-1
// directly, or rows idx[t, a] (gather of the active set) when idx != nullptr.
// --------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void proj_generic_kernel(
    const T* __restrict__ X, int64_t tok_stride, int64_t C, int nvec,
    const int32_t* __restrict__ idx, int Nstreams,
    const float* __restrict__ phiA, int colsA, const float* __restrict__ phiB, int colsB,
    float* __restrict__ P, float* __restrict__ ss) {
  const int64_t t = blockIdx.x;
  const int col0 = blockIdx.y * 32;
  const int ncols = colsA + colsB;
  const int nc = min(32, ncols - col0);
  float acc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) acc[j] = 0.f;
  float sq = 0.f;
  const T* xt = X + t * tok_stride;
  for (int a = 0; a < nvec; ++a) {
    const int s = idx ? idx[t * nvec + a] : a;
    const bool valid = (s >= 0 && s < Nstreams);
    const T* xs = xt + (int64_t)(valid ? s : 0) * C;
    for (int64_t c = threadIdx.x; c < C; c += blockDim.x) {
      const float x = valid ? Elem<T>::ld(xs + c) : 0.f;
      sq += x * x;
      const int64_t row = (int64_t)a * C + c;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (j < nc) {
          const int col = col0 + j;
          const float w = (col < colsA) ? phiA[row * colsA + col] : phiB[row * colsB + (col - colsA)];
          acc[j] += x * w;
        }
      }
    }
  }
  __shared__ float red[4][33];
  __shared__ float redsq[4];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float v = wave_sum(acc[j]);
    if (lane == 0) red[wid][j] = v;
  }
  sq = wave_sum(sq);
  if (lane == 0) redsq[wid] = sq;
  __syncthreads();
  if ((int)threadIdx.x < nc) {
    float s = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += red[w][threadIdx.x];
    P[t * ncols + col0 + threadIdx.x] = s;
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
    float s = 0.f;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) s += redsq[w];
    ss[t] = s;
  }
}

// The same projection when phi is small enough to sit in LDS (nvec C rows x up to
// 32 columns, at most PROJ_LDS_FLOATS with the padding). Each workgroup of 4
// waves stages phi once, row-major with a row stride of ncols + 1 floats, and
// each wave takes tok_per_wave tokens, one at a time: it copies vec(x_t) to its
// own LDS row buffer (and forms ss), then lane (g, j) = (lane >> 5, lane & 31)
// adds x[r] phi[r, j] over half g of the rows, and the two halves of the wave
// are added. One accumulator per lane keeps the code small. At 512 tokens
// of 4 x 256 floats it takes 27 us against 34 us for proj_generic_kernel (the
// staging about 10 us of it, the products about 8); forms with 32 accumulators
// per lane, fully unrolled, took 37-57 us.
constexpr int PROJ_LDS_FLOATS = 25 * 1024;  // 100 KB (4 x 256 rows x 24 columns fit)
constexpr int PROJ_THREADS = 256;
constexpr int PROJ_XMAX = 1024;             // vec(x_t) floats per wave buffer (4 KB)
constexpr int PROJ_SB = 100;                // phi elements per thread per staging batch
constexpr int PROJ_XB = 16;                 // rows of vec(x_t) per lane per batch
template <typename T>
__global__ __launch_bounds__(PROJ_THREADS) void proj_lds_kernel(
    const T* __restrict__ X, int64_t tok_stride, int64_t T_, int64_t C, int nvec,
    const int32_t* __restrict__ idx, int Nstreams,
    const float* __restrict__ phiA, int colsA, const float* __restrict__ phiB, int colsB,
    float* __restrict__ P, float* __restrict__ ss, int tok_per_wave) {
  __shared__ float phs[PROJ_LDS_FLOATS];                    // [R][ncols + 1]
  __shared__ __attribute__((aligned(16))) float xs[PROJ_THREADS / 64][PROJ_XMAX];  // vec(x_t) per wave
  const int ncols = colsA + colsB, RS = ncols + 1;
  const int Ci = (int)C;
  const int R = nvec * Ci;  // (R <= PROJ_XMAX, R * RS <= PROJ_LDS_FLOATS: 32-bit indices)
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  // phi: element e = row * ncols + col of [phiA | phiB] (phiA's elements are
  // consecutive in memory, phiB's too); row = floor((e + 0.5) / ncols), exact in
  // float for e < 2^16 and ncols <= 32
  const int nAB = R * ncols;
  const float inv = 1.0f / (float)ncols;
  for (int e0 = 0; e0 < nAB; e0 += PROJ_SB * PROJ_THREADS) {
    float sv[PROJ_SB];
#pragma unroll
    for (int k = 0; k < PROJ_SB; ++k) {
      const int e = e0 + tid + k * PROJ_THREADS;
      const int ec = e < nAB ? e : nAB - 1;  // (past the end: a valid address, the value unused)
      const int row = (int)(((float)ec + 0.5f) * inv);
      const int col = ec - row * ncols;
      sv[k] = col < colsA ? phiA[row * colsA + col] : phiB[row * colsB + (col - colsA)];
    }
#pragma unroll
    for (int k = 0; k < PROJ_SB; ++k) {
      const int e = e0 + tid + k * PROJ_THREADS;
      const int row = (int)(((float)e + 0.5f) * inv);
      if (e < nAB) phs[row * RS + (e - row * ncols)] = sv[k];
    }
  }
  __syncthreads();
  const int64_t t0 = ((int64_t)blockIdx.x * (PROJ_THREADS >> 6) + wid) * tok_per_wave;
  const int64_t t1 = t0 + tok_per_wave < T_ ? t0 + tok_per_wave : T_;
  float* xw = xs[wid];
  const int g = lane >> 5, j = lane & 31;
  const bool jok = j < ncols;
  for (int64_t t = t0; t < t1; ++t) {
    // vec(x_t) into the wave's buffer (zeros for indices outside [0, Nstreams))
    // (PROJ_XB rows per lane per batch, all loads of a batch in flight first)
    const T* xt = X + t * tok_stride;
    float sq = 0.f;
    for (int r0 = 0; r0 < R; r0 += 64 * PROJ_XB) {
      float xv[PROJ_XB];
#pragma unroll
      for (int u = 0; u < PROJ_XB; ++u) {
        const int r = r0 + lane + 64 * u;
        float x = 0.f;
        if (r < R) {
          const int a = r / Ci;
          const int s = idx ? idx[t * nvec + a] : a;
          if (s >= 0 && s < Nstreams) x = Elem<T>::ld(xt + (int64_t)s * C + (r - a * Ci));
        }
        xv[u] = x;
      }
#pragma unroll
      for (int u = 0; u < PROJ_XB; ++u) {
        const int r = r0 + lane + 64 * u;
        sq += xv[u] * xv[u];
        if (r < R) xw[r] = xv[u];
      }
    }
    __builtin_amdgcn_wave_barrier();  // (one wave's LDS accesses run in order)
    float acc = 0.f;
    if (jok) {  // half g of the rows, 4 at a time (x as one float4, read by the half's lanes alike)
      const int Rh = ((R + 7) >> 3) << 2;  // rows per half, a multiple of 4
      const int rb = g * Rh, re = R < rb + Rh ? R : rb + Rh;
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;  // four partial sums: no single chain of adds
      int r = rb;
#pragma unroll 2
      for (; r + 3 < re; r += 4) {
        const float4 x4 = *reinterpret_cast<const float4*>(xw + r);
        const float* ph = phs + r * RS + j;
        a0 += x4.x * ph[0];
        a1 += x4.y * ph[RS];
        a2 += x4.z * ph[2 * RS];
        a3 += x4.w * ph[3 * RS];
      }
      for (; r < re; ++r) a0 += xw[r] * phs[r * RS + j];
      acc = (a0 + a1) + (a2 + a3);
    }
    acc += __shfl_xor(acc, 32, 64);
    sq = wave_sum(sq);
    if (g == 0 && jok) P[t * ncols + j] = acc;
    if (lane == 0) ss[t] = sq;
    __builtin_amdgcn_wave_barrier();  // the buffer is rewritten by the next token
  }
}

// --------------------------------------------------------------------------
// Coefficient epilogue for 4 x 4 residual maps: 16 lanes per token, 16 tokens per
// workgroup, with the arithmetic of the generic epilogue below (r from ss, the
// gates, the largest logit subtracted before exp, then the iterations of a
// column and a row normalisation), the column and row sums formed by DPP lane
// exchanges within the 16-lane row (lane e = i * 4 + j holds M[i, j]).
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void coeff_epilogue_n4_kernel(
    const float* __restrict__ P, const float* __restrict__ ss, float len, int64_t T_,
    int npre, int npost, float a_pre, float a_post, float a_res, const float* __restrict__ bias, int iters,
    float* __restrict__ h_pre, float* __restrict__ h_post, float* __restrict__ h_res) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t t = g >> 4;
  const int e = (int)(g & 15);
  const bool valid = t < T_;
  const int64_t tc = valid ? t : T_ - 1;
  const int ncols = npre + npost + 16;
  const float* pt = P + tc * ncols;
  const float r = sqrtf(ss[tc] / len);
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  for (int j = e; j < npre; j += 16)
    if (valid && h_pre) h_pre[t * npre + j] = sigmoid(a_pre * (pt[j] * invr) + bias[j]);
  for (int j = e; j < npost; j += 16)
    if (valid) h_post[t * npost + j] = 2.0f * sigmoid(a_post * (pt[npre + j] * invr) + bias[npre + j]);
  const float z = a_res * (pt[npre + npost + e] * invr) + bias[npre + npost + e];
  float zm = fmaxf(z, dpp<DPP_QXOR1>(z));
  zm = fmaxf(zm, dpp<DPP_QXOR2>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR4>(zm));
  zm = fmaxf(zm, dpp<DPP_ROR8>(zm));
  float M = expf(z - zm);
  for (int it = 0; it < iters; ++it) {
    float cs = M + dpp<DPP_ROR8>(M);  // column j: lanes j, j + 4, j + 8, j + 12
    cs += dpp<DPP_ROR4>(cs);
    M = M / cs;
    float rs = M + dpp<DPP_QXOR1>(M);  // row i: the quad 4i .. 4i + 3
    rs += dpp<DPP_QXOR2>(rs);
    M = M / rs;
  }
  if (valid) h_res[t * 16 + e] = M;
}

// --------------------------------------------------------------------------
// Coefficient epilogue, one workgroup (256 threads) per token.
// Logit row P[t] has npre | npost | nres*nres columns. With r = sqrt(ss/len):
//   h_pre  = sigmoid(alpha_pre  * P / r + b)          (mHC notes Eq. 16-17)
//   h_post = 2 sigmoid(alpha_post * P / r + b)        (Eq. 18; xHC post map)
//   h_res  = Sinkhorn-Knopp(exp(alpha_res * P / r + b)) (Eq. 9, 19)
// exp is taken after subtracting the largest logit of the token: a common
// factor of M^(0) that the first column normalisation removes.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(256) void coeff_epilogue_generic_kernel(
    const float* __restrict__ P, const float* __restrict__ ss, float len,
    int npre, int npost, int nres,
    float a_pre, float a_post, float a_res, const float* __restrict__ bias, int iters,
    float* __restrict__ h_pre, float* __restrict__ h_post, float* __restrict__ h_res) {
  const int64_t t = blockIdx.x;
  const int ncols = npre + npost + nres * nres;
  const int nn = nres * nres;
  __shared__ float M[256];
  __shared__ float csum[16], rsum[16];
  __shared__ float red[4];
  const float* pt = P + t * ncols;
  const float r = sqrtf(ss[t] / len);
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  const int tid = threadIdx.x;
  if (tid < npre && h_pre) h_pre[t * npre + tid] = sigmoid(a_pre * (pt[tid] * invr) + bias[tid]);
  for (int j = tid; j < npost; j += blockDim.x)
    h_post[t * npost + j] = 2.0f * sigmoid(a_post * (pt[npre + j] * invr) + bias[npre + j]);
  if (nres == 0) return;
  float z = -INFINITY;
  if (tid < nn) z = a_res * (pt[npre + npost + tid] * invr) + bias[npre + npost + tid];
  // block max of z
  float zm = wave_max(z);
  if ((tid & 63) == 0) red[tid >> 6] = zm;
  __syncthreads();
  zm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (tid < nn) M[tid] = expf(z - zm);
  __syncthreads();
  for (int it = 0; it < iters; ++it) {
    if (tid < nres) {
      float s = 0.f;
      for (int i = 0; i < nres; ++i) s += M[i * nres + tid];
      csum[tid] = s;
    }
    __syncthreads();
    if (tid < nn) M[tid] = M[tid] / csum[tid % nres];
    __syncthreads();
    if (tid < nres) {
      float s = 0.f;
      for (int j = 0; j < nres; ++j) s += M[tid * nres + j];
      rsum[tid] = s;
    }
    __syncthreads();
    if (tid < nn) M[tid] = M[tid] / rsum[tid / nres];
    __syncthreads();
  }
  if (tid < nn) h_res[t * nn + tid] = M[tid];
}

// --------------------------------------------------------------------------
// xHC full-state epilogue + selection, one thread per token.
//   h_pre[i] = sigmoid(alpha_pre * P[i] / r + b_pre[i]), i < N
//   score[j] = sigmoid(P[N + j] / r), candidate stream m + j, j < N - m
//   idx = {0..m-1} U top-(k-m) candidates (ties -> lower index), ascending.
// (xHC summary, sparse residual stream architecture, steps 1-2.)
// --------------------------------------------------------------------------
__global__ __launch_bounds__(64) void xhc_select_kernel(
    const float* __restrict__ P, int pcols, int pre_off, int router_off,
    const float* __restrict__ ss, float len, int64_t T, int N, int k, int m,
    float a_pre, const float* __restrict__ b_pre, float* __restrict__ h_pre,
    float* __restrict__ score, int32_t* __restrict__ idx) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* pt = P + t * pcols;
  const float r = sqrtf(ss[t] / len);
  const float invr = (r > 0.f) ? 1.0f / r : 0.f;
  if (h_pre) {
    for (int i = 0; i < N; ++i) h_pre[t * N + i] = sigmoid(a_pre * (pt[pre_off + i] * invr) + b_pre[i]);
  }
  if (!idx) return;
  const int nc = N - m;
  uint64_t chosen = 0;
  for (int j = 0; j < nc; ++j) {
    const float s = sigmoid(pt[router_off + j] * invr);
    if (score) score[t * nc + j] = s;
  }
  for (int q = 0; q < k - m; ++q) {
    int best = -1;
    float bs = 0.f;
    for (int j = 0; j < nc; ++j) {
      if ((chosen >> j) & 1ull) continue;
      const float s = sigmoid(pt[router_off + j] * invr);
      if (best < 0 || s > bs) { best = j; bs = s; }
    }
    chosen |= 1ull << best;
  }
  int o = 0;
  for (int i = 0; i < m; ++i) idx[t * k + o++] = i;
  for (int j = 0; j < nc; ++j)
    if ((chosen >> j) & 1ull) idx[t * k + o++] = m + j;
}

// --------------------------------------------------------------------------
// Dense pre-read F_in[t, c] = sum_i h[t, i] X[t, i, c] (mHC notes 4.3.1 F_pre;
// xHC summary step 2). One thread per (token, 8 channels).
// --------------------------------------------------------------------------
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void pre_generic_kernel(
    const T* __restrict__ X, int64_t T_, int n, int64_t C, const float* __restrict__ h,
    T* __restrict__ F_in) {
  const int64_t nch = (C + 7) / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T_ * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const int cnt = (int)min((int64_t)8, C - c0);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // rows 4 at a time, all 4 loads issued before use; past n the row index is
  // clamped (no branch around a load) and the row is not added
  for (int i0 = 0; i0 < n; i0 += 4) {
    float x[4][8], w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u < n ? i0 + u : n - 1;
      w[u] = h[t * n + i];
      const T* p = X + (t * n + i) * C + c0;
      if (VEC) load8_nt(p, x[u]); else load8_tail(p, cnt, x[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i0 + u < n) {  // (a padded row times a zero weight could still give NaN)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w[u] * x[u][e];
      }
  }
  T* q = F_in + t * C + c0;
  if (VEC) store8_nt(q, acc); else store8_tail(q, cnt, acc);
}

// --------------------------------------------------------------------------
// Post/res write X_next[t, i] = sum_j h_res[t, i, j] X[t, j] + h_post[t, i] F[t]
// (mHC notes Eq. 3, 4.3.1 F_post,res). One thread per (token, 8 channels); it
// reads all NS rows of its chunk before writing, so X_next may equal X.
// --------------------------------------------------------------------------
template <typename T, int NS, bool VEC>
__global__ __launch_bounds__(256) void post_generic_kernel(
    const T* X, int64_t T_, int64_t C, const float* __restrict__ h_res,
    const float* __restrict__ h_post, const T* __restrict__ F, T* Y) {
  const int64_t nch = (C + 7) / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T_ * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const int cnt = (int)min((int64_t)8, C - c0);
  float x[NS][8], f[8];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const T* p = X + (t * NS + j) * C + c0;
    if (VEC) load8_nt(p, x[j]); else load8_tail(p, cnt, x[j]);
  }
  if (VEC) load8_nt(F + t * C + c0, f); else load8_tail(F + t * C + c0, cnt, f);
  const float* hr = h_res + t * NS * NS;
  const float* hp = h_post + t * NS;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float wp = hp[i];
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = wp * f[e];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const float w = hr[i * NS + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += w * x[j][e];
    }
    T* q = Y + (t * NS + i) * C + c0;
    if (VEC) store8_nt(q, y); else store8_tail(q, cnt, y);
  }
}

// --------------------------------------------------------------------------
// xHC sparse mix + scatter, in place (xHC summary step 3):
//   X[t, idx[a]] = sum_b H_res[t, a, b] X[t, idx[b]] + sum_j H_post[t, a, j] Wb[t, j]
// One thread per (token, 8 channels); all KA gathered rows are read before any
// is written. Tokens with an index outside [0, N) are left unchanged.
// --------------------------------------------------------------------------
template <typename T, int KA, bool VEC>
__global__ __launch_bounds__(256) void mix_generic_kernel(
    T* X, int64_t T_, int N, int64_t C, const int32_t* __restrict__ idx,
    const float* __restrict__ H_res, const float* __restrict__ H_post,
    const T* __restrict__ Wb, int K, const T* __restrict__ Wb2, int j0) {  // rows j >= j0 from Wb2 [T_, K - j0, C]
  const int64_t nch = (C + 7) / 8;
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= T_ * nch) return;
  const int64_t t = g / nch;
  const int64_t c0 = (g - t * nch) * 8;
  const int cnt = (int)min((int64_t)8, C - c0);
  int s[KA];
  bool ok = true;
#pragma unroll
  for (int a = 0; a < KA; ++a) {
    s[a] = idx[t * KA + a];
    ok = ok && (s[a] >= 0 && s[a] < N);
  }
  if (!ok) return;
  float x[KA][8];
#pragma unroll
  for (int a = 0; a < KA; ++a) {
    const T* p = X + (t * N + s[a]) * C + c0;
    if (VEC) load8(p, x[a]); else load8_tail(p, cnt, x[a]);
  }
  float y[KA][8];
  const float* hr = H_res + t * KA * KA;
  const float* hp = H_post + t * KA * K;
#pragma unroll
  for (int a = 0; a < KA; ++a) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[a][e] = 0.f;
#pragma unroll
    for (int b = 0; b < KA; ++b) {
      const float w = hr[a * KA + b];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[a][e] += w * x[b][e];
    }
  }
  for (int j = 0; j < K; ++j) {
    float wv[8];
    const T* p = j < j0 ? Wb + (t * K + j) * C + c0 : Wb2 + (t * (K - j0) + (j - j0)) * C + c0;
    if (VEC) load8(p, wv); else load8_tail(p, cnt, wv);
#pragma unroll
    for (int a = 0; a < KA; ++a) {
      const float w = hp[a * K + j];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[a][e] += w * wv[e];
    }
  }
#pragma unroll
  for (int a = 0; a < KA; ++a) {
    T* q = X + (t * N + s[a]) * C + c0;
    if (VEC) store8(q, y[a]); else store8_tail(q, cnt, y[a]);
  }
}

// --------------------------------------------------------------------------
// Temporal augmentation, one workgroup per token (xHC summary, temporal
// feature augmentation): causal depthwise convs, then Gram-Schmidt in the
// modified form. The K_r components of the token live in LDS as float32.
// --------------------------------------------------------------------------
template <typename T, typename TV>
__global__ __launch_bounds__(256) void augment_generic_kernel(
    const T* __restrict__ F, int64_t S, int64_t C, const float* __restrict__ w,
    ConvSpec spec, TV* __restrict__ V) {
  extern __shared__ float comps[];  // [Kr][C]
  __shared__ float red[4];
  __shared__ float norms[HC_MAX_COMPONENTS_DEV];
  const int64_t t = blockIdx.x;
  const int64_t pos = t % S;  // position inside its sequence
  const int Kr = spec.r + 1;
  for (int64_t c = threadIdx.x; c < C; c += blockDim.x) comps[c] = Elem<T>::ld(F + t * C + c);
  for (int j = 0; j < spec.r; ++j) {
    const int kap = spec.kappa[j];
    const float* wj = w + spec.offset[j];
    for (int64_t c = threadIdx.x; c < C; c += blockDim.x) {
      float g = 0.f;
      for (int s = 0; s < kap; ++s) {
        const int64_t src = pos - kap + 1 + s;
        if (src >= 0) g += wj[c * kap + s] * Elem<T>::ld(F + (t - pos + src) * C + c);
      }
      comps[(j + 1) * C + c] = g;
    }
  }
  __syncthreads();
  for (int j = 1; j < Kr; ++j) {
    if (j - 1 >= 0) {
      // squared norm of the finished component j-1
      float p = 0.f;
      for (int64_t c = threadIdx.x; c < C; c += blockDim.x) {
        const float v = comps[(j - 1) * C + c];
        p += v * v;
      }
      const float nv = block_sum(p, red);
      if (threadIdx.x == 0) norms[j - 1] = nv;
    }
    for (int i = 0; i < j; ++i) {
      float p = 0.f;
      for (int64_t c = threadIdx.x; c < C; c += blockDim.x) p += comps[j * C + c] * comps[i * C + c];
      const float num = block_sum(p, red);
      __syncthreads();
      const float coef = num / norms[i];
      for (int64_t c = threadIdx.x; c < C; c += blockDim.x) comps[j * C + c] -= coef * comps[i * C + c];
      __syncthreads();
    }
  }
  __syncthreads();
  for (int j = 0; j < Kr; ++j)
    for (int64_t c = threadIdx.x; c < C; c += blockDim.x)
      Elem<TV>::st(V + (t * Kr + j) * C + c, comps[j * C + c]);
}

// ==========================================================================
// Host-side launchers
// ==========================================================================

static inline unsigned grid1(int64_t work, int block) { return (unsigned)((work + block - 1) / block); }

template <typename T>
static hipError_t launch_proj_t(const void* X, int64_t tok_stride, int64_t T_, int64_t C, int nvec,
                                const int32_t* idx, int Nstreams, const float* phiA, int colsA,
                                const float* phiB, int colsB, float* P, float* ss, hipStream_t st) {
  const int ncols = colsA + colsB;
  if (ncols <= 32 && (int64_t)nvec * C <= PROJ_XMAX && (int64_t)nvec * C * (ncols + 1) <= PROJ_LDS_FLOATS) {
    // each wave takes tok_per_wave tokens; one workgroup (of 4 waves) per CU
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 1)
      ncu = 256;
    const int64_t waves = 4 * (int64_t)ncu;
    const int tpw = (int)((T_ + waves - 1) / waves);
    const int64_t nwg = (T_ + 4 * (int64_t)tpw - 1) / (4 * (int64_t)tpw);
    hipLaunchKernelGGL(proj_lds_kernel<T>, dim3((unsigned)nwg), dim3(PROJ_THREADS), 0, st, (const T*)X, tok_stride,
                       T_, C, nvec, idx, Nstreams, phiA, colsA, phiB, colsB, P, ss, tpw);
    return hipGetLastError();
  }
  dim3 grid((unsigned)T_, (unsigned)((ncols + 31) / 32));
  hipLaunchKernelGGL(proj_generic_kernel<T>, grid, dim3(256), 0, st, (const T*)X, tok_stride, C,
                     nvec, idx, Nstreams, phiA, colsA, phiB, colsB, P, ss);
  return hipGetLastError();
}

hipError_t launch_proj_generic(int dtype, const void* X, int64_t tok_stride, int64_t T_, int64_t C,
                               int nvec, const int32_t* idx, int Nstreams, const float* phiA,
                               int colsA, const float* phiB, int colsB, float* P, float* ss,
                               hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  if (dtype == 0)
    return launch_proj_t<float>(X, tok_stride, T_, C, nvec, idx, Nstreams, phiA, colsA, phiB, colsB, P, ss, st);
  return launch_proj_t<bf16_t>(X, tok_stride, T_, C, nvec, idx, Nstreams, phiA, colsA, phiB, colsB, P, ss, st);
}

hipError_t launch_coeff_epilogue(const float* P, const float* ss, float len, int64_t T_, int npre,
                                 int npost, int nres, float a_pre, float a_post, float a_res,
                                 const float* bias, int iters, float* h_pre, float* h_post,
                                 float* h_res, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  if (nres == 4) {
    hipLaunchKernelGGL(coeff_epilogue_n4_kernel, dim3(grid1(T_ * 16, 256)), dim3(256), 0, st, P, ss, len, T_, npre,
                       npost, a_pre, a_post, a_res, bias, iters, h_pre, h_post, h_res);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(coeff_epilogue_generic_kernel, dim3((unsigned)T_), dim3(256), 0, st, P, ss, len,
                     npre, npost, nres, a_pre, a_post, a_res, bias, iters, h_pre, h_post, h_res);
  return hipGetLastError();
}

hipError_t launch_xhc_select(const float* P, int pcols, int pre_off, int router_off, const float* ss,
                             float len, int64_t T_, int N, int k, int m, float a_pre,
                             const float* b_pre, float* h_pre, float* score, int32_t* idx,
                             hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  hipLaunchKernelGGL(xhc_select_kernel, dim3(grid1(T_, 64)), dim3(64), 0, st, P, pcols, pre_off,
                     router_off, ss, len, T_, N, k, m, a_pre, b_pre, h_pre, score, idx);
  return hipGetLastError();
}

hipError_t launch_pre_generic(int dtype, bool vec, const void* X, int64_t T_, int n, int64_t C,
                              const float* h, void* F_in, hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  const int64_t work = T_ * ((C + 7) / 8);
  const dim3 g(grid1(work, 256)), b(256);
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((pre_generic_kernel<float, true>), g, b, 0, st, (const float*)X, T_, n, C, h, (float*)F_in);
    else hipLaunchKernelGGL((pre_generic_kernel<float, false>), g, b, 0, st, (const float*)X, T_, n, C, h, (float*)F_in);
  } else {
    if (vec) hipLaunchKernelGGL((pre_generic_kernel<bf16_t, true>), g, b, 0, st, (const bf16_t*)X, T_, n, C, h, (bf16_t*)F_in);
    else hipLaunchKernelGGL((pre_generic_kernel<bf16_t, false>), g, b, 0, st, (const bf16_t*)X, T_, n, C, h, (bf16_t*)F_in);
  }
  return hipGetLastError();
}

template <typename T, int NS>
static void post_dispatch_vec(bool vec, const void* X, int64_t T_, int64_t C, const float* h_res,
                              const float* h_post, const void* F, void* Y, hipStream_t st) {
  const int64_t work = T_ * ((C + 7) / 8);
  const dim3 g(grid1(work, 256)), b(256);
  if (vec)
    hipLaunchKernelGGL((post_generic_kernel<T, NS, true>), g, b, 0, st, (const T*)X, T_, C, h_res, h_post, (const T*)F, (T*)Y);
  else
    hipLaunchKernelGGL((post_generic_kernel<T, NS, false>), g, b, 0, st, (const T*)X, T_, C, h_res, h_post, (const T*)F, (T*)Y);
}

template <typename T>
static void post_dispatch_n(int n, bool vec, const void* X, int64_t T_, int64_t C,
                            const float* h_res, const float* h_post, const void* F, void* Y,
                            hipStream_t st) {
  switch (n) {
#define HC_POST_CASE(NS) \
  case NS: post_dispatch_vec<T, NS>(vec, X, T_, C, h_res, h_post, F, Y, st); break;
    HC_POST_CASE(1) HC_POST_CASE(2) HC_POST_CASE(3) HC_POST_CASE(4)
    HC_POST_CASE(5) HC_POST_CASE(6) HC_POST_CASE(7) HC_POST_CASE(8)
    HC_POST_CASE(9) HC_POST_CASE(10) HC_POST_CASE(11) HC_POST_CASE(12)
    HC_POST_CASE(13) HC_POST_CASE(14) HC_POST_CASE(15) HC_POST_CASE(16)
#undef HC_POST_CASE
    default: break;
  }
}

hipError_t launch_post_generic(int dtype, bool vec, const void* X, int64_t T_, int n, int64_t C,
                               const float* h_res, const float* h_post, const void* F, void* Y,
                               hipStream_t st) {
  if (T_ == 0) return hipSuccess;
  if (dtype == 0) post_dispatch_n<float>(n, vec, X, T_, C, h_res, h_post, F, Y, st);
  else post_dispatch_n<bf16_t>(n, vec, X, T_, C, h_res, h_post, F, Y, st);
  return hipGetLastError();
}

template <typename T, int KA>
static void mix_dispatch_vec(bool vec, void* X, int64_t T_, int N, int64_t C, const int32_t* idx,
                             const float* H_res, const float* H_post, const void* Wb, int K,
                             hipStream_t st, const void* Wb2, int j0) {
  const int64_t work = T_ * ((C + 7) / 8);
  const dim3 g(grid1(work, 256)), b(256);
  if (vec)
    hipLaunchKernelGGL((mix_generic_kernel<T, KA, true>), g, b, 0, st, (T*)X, T_, N, C, idx, H_res, H_post, (const T*)Wb, K,
                       (const T*)Wb2, j0);
  else
    hipLaunchKernelGGL((mix_generic_kernel<T, KA, false>), g, b, 0, st, (T*)X, T_, N, C, idx, H_res, H_post, (const T*)Wb, K,
                       (const T*)Wb2, j0);
}

template <typename T>
static void mix_dispatch_k(int k, bool vec, void* X, int64_t T_, int N, int64_t C,
                           const int32_t* idx, const float* H_res, const float* H_post,
                           const void* Wb, int K, hipStream_t st, const void* Wb2, int j0) {
  switch (k) {
#define HC_MIX_CASE(KA) \
  case KA: mix_dispatch_vec<T, KA>(vec, X, T_, N, C, idx, H_res, H_post, Wb, K, st, Wb2, j0); break;
    HC_MIX_CASE(1) HC_MIX_CASE(2) HC_MIX_CASE(3) HC_MIX_CASE(4)
    HC_MIX_CASE(5) HC_MIX_CASE(6) HC_MIX_CASE(7) HC_MIX_CASE(8)
    HC_MIX_CASE(9) HC_MIX_CASE(10) HC_MIX_CASE(11) HC_MIX_CASE(12)
    HC_MIX_CASE(13) HC_MIX_CASE(14) HC_MIX_CASE(15) HC_MIX_CASE(16)
#undef HC_MIX_CASE
    default: break;
  }
}

hipError_t launch_mix_generic(int dtype, bool vec, void* X, int64_t T_, int N, int64_t C, int k,
                              const int32_t* idx, const float* H_res, const float* H_post,
                              const void* Wb, int K, hipStream_t st, const void* Wb2, int j0) {
  if (T_ == 0) return hipSuccess;
  if (!Wb2) j0 = K;
  if (dtype == 0) mix_dispatch_k<float>(k, vec, X, T_, N, C, idx, H_res, H_post, Wb, K, st, Wb2, j0);
  else mix_dispatch_k<bf16_t>(k, vec, X, T_, N, C, idx, H_res, H_post, Wb, K, st, Wb2, j0);
  return hipGetLastError();
}

int64_t augment_generic_lds_bytes(int r, int64_t C) { return (int64_t)(r + 1) * C * 4; }

hipError_t launch_augment_generic(int dtype, int vdtype, const void* F, int64_t B, int64_t S,
                                  int64_t C, const float* w, const ConvSpec& spec, void* V,
                                  hipStream_t st) {
  const int64_t T_ = B * S;
  if (T_ == 0) return hipSuccess;
  const size_t lds = (size_t)augment_generic_lds_bytes(spec.r, C);
  const dim3 g((unsigned)T_), b(256);
  if (dtype == 0 && vdtype == 0)
    hipLaunchKernelGGL((augment_generic_kernel<float, float>), g, b, lds, st, (const float*)F, S, C, w, spec, (float*)V);
  else if (dtype == 0 && vdtype == 1)
    hipLaunchKernelGGL((augment_generic_kernel<float, bf16_t>), g, b, lds, st, (const float*)F, S, C, w, spec, (bf16_t*)V);
  else if (dtype == 1 && vdtype == 0)
    hipLaunchKernelGGL((augment_generic_kernel<bf16_t, float>), g, b, lds, st, (const bf16_t*)F, S, C, w, spec, (float*)V);
  else
    hipLaunchKernelGGL((augment_generic_kernel<bf16_t, bf16_t>), g, b, lds, st, (const bf16_t*)F, S, C, w, spec, (bf16_t*)V);
  return hipGetLastError();
}

}  // namespace hc
