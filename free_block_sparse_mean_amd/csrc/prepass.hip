// Block-summary pre-pass for Sol-Attn on gfx950.
//
// Reads K and V once and produces what the fused pass needs to route every
// query block without forming a row of proxy scores:
//   k_bar_j = mean of the 64 keys of block j         (row-major and transposed)
//   vsum_j  = sum of the 64 values of block j        (= 64 * v_bar_j)
//   m       = mean over j of k_bar_j
//   C       = (1/n_b) sum_j (k_bar_j - m)(k_bar_j - m)^T   (centred, population)
// Sources: page "Sol-Attn: l'attenzione sparsa che sceglie al volo"
// (paithon.it), section "Perche l'attenzione pesa tanto nei video" for the
// 64-token block means, section "Una soglia per ogni riga" (last paragraph)
// for mu_i/sigma_i from the key-summary mean and d x d second moments, and
// section "Scegliere mentre si calcola" for the block-mean values the
// correction reuses.
//
// Bound: HBM bandwidth. block_sums streams 2*N*d input elements per head with
// 16-byte loads, one wave per block; the mean/covariance kernels touch only
// the n_b x d summaries (L2-resident) and accumulate in double so that the
// closed-form threshold carries no cancellation from the key mean.
#include "device_common.hpp"
#include "sol_internal.hpp"

namespace sol {
namespace {

// One wave per key block: lane (rg, cc) sums rows rg, rg+RG, ... of 16-byte
// column chunk cc for K and V, then the row groups are folded by xor-shuffles.
template <typename T, int D>
__global__ __launch_bounds__(256) void block_sums_kernel(const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         float* __restrict__ kbar,
                                                         float* __restrict__ vsum,
                                                         int n_b, long long N) {
  using V = Vec16<T>;
  constexpr int E = V::kN;     // elements per 16-byte chunk
  constexpr int CH = D / E;    // chunks per row
  constexpr int RG = 64 / CH;  // row groups
  constexpr int RPL = 64 / RG; // rows per lane
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long bh = blockIdx.y;
  if (j >= n_b) return;
  const int cc = lane % CH, rg = lane / CH;
  const size_t base = ((size_t)bh * N + (size_t)j * kBlock) * D;
  const typename V::raw* pk = reinterpret_cast<const typename V::raw*>(k + base) + cc;
  const typename V::raw* pv = reinterpret_cast<const typename V::raw*>(v + base) + cc;
  float ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { ak[e] = 0.f; av[e] = 0.f; }
#pragma unroll 8
  for (int i = 0; i < RPL; ++i) {
    const int r = rg + RG * i;
    float fk[E], fv[E];
    V::to_float(pk[(size_t)r * CH], fk);
    V::to_float(pv[(size_t)r * CH], fv);
#pragma unroll
    for (int e = 0; e < E; ++e) { ak[e] += fk[e]; av[e] += fv[e]; }
  }
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      ak[e] += __shfl_xor(ak[e], o, 64);
      av[e] += __shfl_xor(av[e], o, 64);
    }
  }
  if (rg == 0) {
    float* kb = kbar + ((size_t)bh * n_b + j) * D + cc * E;
    float* vs = vsum + ((size_t)bh * n_b + j) * D + cc * E;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kb[e] = ak[e] * (1.0f / kBlock);   // exact scaling by a power of two
      vs[e] = av[e];
    }
  }
}

// m = mean_j k_bar_j per head, accumulated in double.
template <int D>
__global__ __launch_bounds__(256) void key_mean_kernel(const float* __restrict__ kbar,
                                                       float* __restrict__ kmean,
                                                       double* __restrict__ kmean64, int n_b) {
  constexpr int P = 256 / D;
  __shared__ double red[256];
  const int t = threadIdx.x, c = t % D, p = t / D;
  const long long bh = blockIdx.x;
  const float* kb = kbar + (size_t)bh * n_b * D;
  double acc = 0.0;
  for (int j = p; j < n_b; j += P) acc += (double)kb[(size_t)j * D + c];
  red[t] = acc;
  __syncthreads();
  if (t < D) {
    double s = 0.0;
#pragma unroll
    for (int q = 0; q < P; ++q) s += red[q * D + t];
    const double m = s / (double)n_b;
    kmean64[(size_t)bh * D + t] = m;
    kmean[(size_t)bh * D + t] = (float)m;
  }
}

// Partial centred second moments over one chunk of kCovChunk key blocks, in
// double; also writes the transposed summaries kbar_t for the chunk.
template <int D>
__global__ __launch_bounds__(256) void cov_partial_kernel(const float* __restrict__ kbar,
                                                          const double* __restrict__ kmean64,
                                                          float* __restrict__ kbar_t,
                                                          double* __restrict__ cov_part,
                                                          int n_b, int n_b_pad, int parts) {
  constexpr int TJ = 32;       // key blocks staged per step
  constexpr int R = D / 16;    // outputs per thread along each dimension
  __shared__ float tile[TJ][D + 1];
  __shared__ double mloc[D];
  const int t = threadIdx.x, ty = t / 16, tx = t % 16;
  const long long bh = blockIdx.y;
  const int part = blockIdx.x;
  const int j0 = part * kCovChunk;
  const int j1 = min(n_b, j0 + kCovChunk);
  if (t < D) mloc[t] = kmean64[(size_t)bh * D + t];
  double acc[R][R];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < R; ++s) acc[r][s] = 0.0;

  for (int jb = j0; jb < j1; jb += TJ) {
    __syncthreads();
    for (int e = t; e < TJ * D; e += 256) {
      const int jj = e / D, c = e % D, j = jb + jj;
      tile[jj][c] = j < j1 ? kbar[((size_t)bh * n_b + j) * D + c] : 0.f;
    }
    __syncthreads();
    for (int e = t; e < TJ * D; e += 256) {
      const int c = e / TJ, jj = e % TJ, j = jb + jj;
      if (j < j1) kbar_t[((size_t)bh * D + c) * n_b_pad + j] = tile[jj][c];
    }
    const int nj = min(TJ, j1 - jb);
    for (int jj = 0; jj < nj; ++jj) {
      double a[R], b[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        a[r] = (double)tile[jj][ty * R + r] - mloc[ty * R + r];
        b[r] = (double)tile[jj][tx * R + r] - mloc[tx * R + r];
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int s = 0; s < R; ++s) acc[r][s] += a[r] * b[s];
    }
  }
  // zero the row padding of kbar_t once per head
  if (part == parts - 1) {
    for (int e = t; e < D * (n_b_pad - n_b); e += 256) {
      const int c = e / (n_b_pad - n_b), j = n_b + e % (n_b_pad - n_b);
      kbar_t[((size_t)bh * D + c) * n_b_pad + j] = 0.f;
    }
  }
  double* outp = cov_part + ((size_t)bh * parts + part) * D * D;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < R; ++s) outp[(size_t)(ty * R + r) * D + tx * R + s] = acc[r][s];
}

// C = (sum of the partials in chunk order) / n_b, stored as float.
template <int D>
__global__ __launch_bounds__(256) void cov_reduce_kernel(const double* __restrict__ cov_part,
                                                         float* __restrict__ kcov, int n_b,
                                                         int parts) {
  const long long bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  double s = 0.0;
  for (int p = 0; p < parts; ++p) s += cov_part[((size_t)bh * parts + p) * D * D + e];
  kcov[(size_t)bh * D * D + e] = (float)(s / (double)n_b);
}

template <typename T, int D>
hipError_t prepass_impl(const Shape& s, const void* k, const void* v, const Workspace& ws,
                        hipStream_t st) {
  const unsigned bh = (unsigned)s.BH();
  hipLaunchKernelGGL((block_sums_kernel<T, D>), dim3((s.n_b + 3) / 4, bh), dim3(256), 0, st,
                     static_cast<const T*>(k), static_cast<const T*>(v), ws.kbar, ws.vsum, s.n_b,
                     (long long)s.N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((key_mean_kernel<D>), dim3(bh), dim3(256), 0, st, ws.kbar, ws.kmean,
                     ws.kmean64, s.n_b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((cov_partial_kernel<D>), dim3(s.cov_parts, bh), dim3(256), 0, st, ws.kbar,
                     ws.kmean64, ws.kbar_t, ws.cov_part, s.n_b, s.n_b_pad, s.cov_parts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((cov_reduce_kernel<D>), dim3((D * D + 255) / 256, bh), dim3(256), 0, st,
                     ws.cov_part, ws.kcov, s.n_b, s.cov_parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepass(const Shape& s, Dtype dt, const void* k, const void* v,
                          const Workspace& ws, hipStream_t stream) {
  if (dt == Dtype::BF16)
    return s.d == 64 ? prepass_impl<__bf16, 64>(s, k, v, ws, stream)
                     : prepass_impl<__bf16, 128>(s, k, v, ws, stream);
  return s.d == 64 ? prepass_impl<float, 64>(s, k, v, ws, stream)
                   : prepass_impl<float, 128>(s, k, v, ws, stream);
}

}  // namespace sol
