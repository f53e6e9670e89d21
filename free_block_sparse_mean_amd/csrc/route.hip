// Routing baselines with a materialized proxy map, for the routing-cost and
// budget study: the proxy map s_hat = Q_bar K_bar^T / sqrt(d) of every head is
// written to HBM, then each row is selected by
//   * the threshold tau_i = mu_i + beta*sigma_i with mu_i, sigma_i taken from
//     the materialized row (two passes), the strict test s_hat_ij > tau_i;
//   * top-k: the row's k highest scores;
//   * top-p: the best blocks until the softmax probability of the row reaches p.
// Sources: page "Sol-Attn: l'attenzione sparsa che sceglie al volo, per
// generare video piu in fretta" (paithon.it), section "Perche l'attenzione
// pesa tanto nei video" (top-k and top-p over the block-mean proxy, and that
// both build the full score map and the chosen indices in GPU memory before
// attention starts) and section "Una soglia per ogni riga" (the threshold).
// The fused kernel never builds this map; these kernels exist to measure what
// it avoids.
//
// Bounds: qbar_kernel reads Q once (HBM); proxy_map_kernel is an fp32 product
// of n_b x d by d x n_b per head writing n_b^2 floats (VALU and HBM write);
// route_select_kernel reads each row once and sorts it in LDS (top-k, top-p).
#include "device_common.hpp"
#include "sol_internal.hpp"

namespace sol {
namespace {

// One wave per query block: q_bar = mean of its 64 rows (fp32 sums of the
// 16-byte chunks, xor-shuffle folds, then / 64).
template <typename T, int D>
__global__ __launch_bounds__(256) void qbar_kernel(const T* __restrict__ q, float* __restrict__ qbar,
                                                   int n_b, int H, TStrides qs) {
  using V = Vec16<T>;
  constexpr int E = V::kN, CH = D / E, RG = 64 / CH, RPL = 64 / RG;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int i = blockIdx.x * 4 + wv;
  const long long bh = blockIdx.y;
  if (i >= n_b) return;   // whole wave leaves; no barrier in this kernel
  const int cc = lane % CH, rg = lane / CH;
  const T* q0 = q + (bh / H) * qs.b + (bh % H) * qs.h + (long long)i * kBlock * qs.n;   // row 0 of block i
  float a[E];
#pragma unroll
  for (int e = 0; e < E; ++e) a[e] = 0.f;
#pragma unroll 8
  for (int r = 0; r < RPL; ++r) {
    float f[E];
    V::to_float(reinterpret_cast<const typename V::raw*>(q0 + (long long)(rg + RG * r) * qs.n)[cc], f);
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] += f[e];
  }
#pragma unroll
  for (int o = CH; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] += __shfl_xor(a[e], o, 64);
  if (lane < CH)
#pragma unroll
    for (int e = 0; e < E; ++e) qbar[((size_t)bh * n_b + i) * D + cc * E + e] = a[e] * (1.0f / kBlock);
}

// map[bh][i][j] = (sum_c qbar[i][c] kbar[j][c]) / sqrt(d), dims summed in
// ascending order (one fp32 FMA chain per entry). A workgroup computes a
// 128 x 128 tile, 8 x 8 entries per lane (rows 8ty.., columns 8tx..), from
// chunks of 16 head dims of both operands staged in LDS transposed ([c][128],
// so a lane's eight rows or columns are two 16-byte reads); 64 FMAs per four
// LDS reads. Rows and columns past n_b are computed on zeros and not stored.
template <int D>
__global__ __launch_bounds__(256) void proxy_map_kernel(const float* __restrict__ qbar,
                                                        const float* __restrict__ kbar,
                                                        float* __restrict__ map, int n_b) {
  constexpr int TC = 16;          // head dims per staged chunk
  constexpr int PT = 128 + 4;     // pitch of a staged row of 128 entries
  __shared__ __attribute__((aligned(16))) float qs[TC * PT];
  __shared__ __attribute__((aligned(16))) float ks[TC * PT];
  const long long bh = blockIdx.z;
  const int i0 = blockIdx.y * 128, j0 = blockIdx.x * 128, t = threadIdx.x;
  const float* qb = qbar + (size_t)bh * n_b * D;
  const float* kb = kbar + (size_t)bh * n_b * D;
  const int ty = t / 16, tx = t % 16;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
  // staging: lane t loads float4 (row t / 4 + 64 h, dims 4 (t % 4) ..) of both operands
  const int sr = t / 4, sc = 4 * (t % 4);
  for (int c0 = 0; c0 < D; c0 += TC) {
    float4 x[2], y[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = sr + 64 * h;
      x[h] = i0 + r < n_b ? *reinterpret_cast<const float4*>(qb + (size_t)(i0 + r) * D + c0 + sc)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
      y[h] = j0 + r < n_b ? *reinterpret_cast<const float4*>(kb + (size_t)(j0 + r) * D + c0 + sc)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();   // the previous chunk has been read
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = sr + 64 * h;
      qs[(sc + 0) * PT + r] = x[h].x; qs[(sc + 1) * PT + r] = x[h].y;
      qs[(sc + 2) * PT + r] = x[h].z; qs[(sc + 3) * PT + r] = x[h].w;
      ks[(sc + 0) * PT + r] = y[h].x; ks[(sc + 1) * PT + r] = y[h].y;
      ks[(sc + 2) * PT + r] = y[h].z; ks[(sc + 3) * PT + r] = y[h].w;
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < TC; ++c) {
      const float4 q0 = *reinterpret_cast<const float4*>(qs + c * PT + 8 * ty);
      const float4 q1 = *reinterpret_cast<const float4*>(qs + c * PT + 8 * ty + 4);
      const float4 k0 = *reinterpret_cast<const float4*>(ks + c * PT + 8 * tx);
      const float4 k1 = *reinterpret_cast<const float4*>(ks + c * PT + 8 * tx + 4);
      const float qv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const float kv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = fmaf(qv[a], kv[b], acc[a][b]);
    }
  }
  const float scale = D == 64 ? 0.125f : 0.08838834764831845f;
  const int j = j0 + 8 * tx;
  // 16-byte stores where every row starts 16-byte aligned
  const bool vec = (n_b & 3) == 0 && (reinterpret_cast<uintptr_t>(map) & 15) == 0;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = i0 + 8 * ty + a;
    if (i >= n_b) continue;
    float* row = map + ((size_t)bh * n_b + i) * n_b;
    if (vec && j + 8 <= n_b) {
      *reinterpret_cast<float4*>(row + j) =
          make_float4(acc[a][0] * scale, acc[a][1] * scale, acc[a][2] * scale, acc[a][3] * scale);
      *reinterpret_cast<float4*>(row + j + 4) =
          make_float4(acc[a][4] * scale, acc[a][5] * scale, acc[a][6] * scale, acc[a][7] * scale);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        if (j + b < n_b) row[j + b] = acc[a][b] * scale;
    }
  }
}

// Workgroup sum of one float per thread (4 waves); every thread gets the total.
__device__ inline float wg_sum(float x, float* red) {
  x = wave_sum(x);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Ascending order of the 32-bit pattern matches ascending float order.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per row of the map. MODE: kRouteThreshold, kRouteTopK, kRouteTopP.
template <int MODE>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ map, int n_b,
                                                           int n_words, float beta, int beta_mode,
                                                           int topk, float topp,
                                                           uint64_t* __restrict__ mask,
                                                           int32_t* __restrict__ kept,
                                                           int32_t* __restrict__ idx) {
  __shared__ unsigned long long keys[kMaxBlocks];   // (descending score, ascending j) sort keys
  __shared__ float cum[kMaxBlocks];                 // top-p: weights, then prefix sums
  __shared__ unsigned char flag[kMaxBlocks];        // kept blocks of the row
  __shared__ float red[8];
  __shared__ int cut;
  const long long row = blockIdx.x;   // bh * n_b + i
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const float* x = map + (size_t)row * n_b;
  int n_kept = 0;

  if constexpr (MODE == kRouteThreshold) {
    // the row is read once into registers: lane t holds entries t + 256 k,
    // which are also the entries it tests for mask word 4 k + (its wave);
    // mu and sigma of the materialized row (two passes over the registers),
    // tau, strict test
    constexpr int C = kMaxBlocks / 256;
    float xv[C];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const int j = t + 256 * k;
      xv[k] = j < n_b ? x[j] : 0.f;
      s += xv[k];
    }
    const float mu = wg_sum(s, red) / (float)n_b;
    float v = 0.f;
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const float e = xv[k] - mu;
      if (t + 256 * k < n_b) v = fmaf(e, e, v);
    }
    const float sigma = sqrtf(wg_sum(v, red + 4) / (float)n_b);
    const float tau = beta_mode == kBetaMinusInf ? -INFINITY
                      : beta_mode == kBetaPlusInf ? INFINITY
                                                  : mu + beta * sigma;
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const int wi = 4 * k + w, j = wi * 64 + lane;   // = t + 256 k
      if (wi < n_words) {                             // uniform over the wave
        const uint64_t word = __ballot(j < n_b && xv[k] > tau);
        if (lane == 0) mask[(size_t)row * n_words + wi] = word;
        n_kept += (lane == 0) ? __popcll(word) : 0;
      }
    }
    n_kept = (int)wg_sum((float)n_kept, red);
  } else {
    // sort the row by descending score (ties: ascending j) with a bitonic network
    int n = 1;
    while (n < n_b) n <<= 1;
    for (int j = t; j < n; j += 256) {
      keys[j] = j < n_b ? ((unsigned long long)(~ordered_bits(x[j])) << 32) | (unsigned)j : ~0ull;
      flag[j] = 0;
    }
    __syncthreads();
    for (int k = 2; k <= n; k <<= 1) {
      for (int st = k >> 1; st > 0; st >>= 1) {
        for (int i = t; i < n; i += 256) {
          const int p = i ^ st;
          if (p > i) {
            const unsigned long long a = keys[i], b = keys[p];
            if ((a > b) == ((i & k) == 0)) { keys[i] = b; keys[p] = a; }
          }
        }
        __syncthreads();
      }
    }
    if constexpr (MODE == kRouteTopK) {
      n_kept = topk < n_b ? (topk > 0 ? topk : 0) : n_b;
    } else {
      // probabilities in sorted order: w_r = exp(s_r - s_max); cut at the
      // first prefix whose sum reaches p * (total)
      const float smax = x[(int)(keys[0] & 0xFFFFFFFFu)];
      constexpr int C = kMaxBlocks / 256;   // positions per thread (contiguous chunk)
      const int r0 = t * C;
      float part = 0.f;
      for (int r = r0; r < r0 + C && r < n_b; ++r) {
        const float wr = expf(x[(int)(keys[r] & 0xFFFFFFFFu)] - smax);
        cum[r] = wr;
        part += wr;
      }
      // exclusive scan of the 256 chunk sums: within the wave, then across waves
      float incl = part;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      if (t == 0) cut = n_b - 1;
      __syncthreads();
      if (lane == 63) red[w] = incl;
      __syncthreads();
      float base = 0.f;
      for (int q = 0; q < w; ++q) base += red[q];
      const float total = (red[0] + red[1]) + (red[2] + red[3]);
      float run = base + incl - part;
      const float target = topp * total;
      for (int r = r0; r < r0 + C && r < n_b; ++r) {
        run += cum[r];
        if (run >= target) { atomicMin(&cut, r); break; }
      }
      __syncthreads();
      n_kept = cut + 1;
    }
    for (int r = t; r < n_kept; r += 256) {
      const int j = (int)(keys[r] & 0xFFFFFFFFu);
      flag[j] = 1;
      if (MODE == kRouteTopK && idx) idx[(size_t)row * topk + r] = j;
    }
    __syncthreads();
    for (int wi = w; wi < n_words; wi += 4) {
      const int j = wi * 64 + lane;
      const uint64_t word = __ballot(j < n_b && flag[j]);
      if (lane == 0) mask[(size_t)row * n_words + wi] = word;
    }
  }
  if (kept && t == 0) kept[row] = n_kept;
}

template <typename T, int D>
hipError_t route_impl(const Shape& s, const RouteArgs& a, hipStream_t st) {
  const unsigned bh = (unsigned)s.BH();
  hipLaunchKernelGGL((qbar_kernel<T, D>), dim3((s.n_b + 3) / 4, bh), dim3(256), 0, st,
                     static_cast<const T*>(a.q), a.ws.qbar, s.n_b, s.H, a.qs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned tiles = (unsigned)((s.n_b + 127) / 128);
  hipLaunchKernelGGL((proxy_map_kernel<D>), dim3(tiles, tiles, bh), dim3(256), 0, st, a.ws.qbar,
                     a.ws.kbar, a.proxy_map, s.n_b);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 grid((unsigned)(s.BH() * s.n_b));
  if (a.mode == kRouteThreshold)
    hipLaunchKernelGGL((route_select_kernel<kRouteThreshold>), grid, dim3(256), 0, st, a.proxy_map, s.n_b,
                       s.n_words, a.beta, a.beta_mode, 0, 0.f, a.mask, a.kept, a.idx);
  else if (a.mode == kRouteTopK)
    hipLaunchKernelGGL((route_select_kernel<kRouteTopK>), grid, dim3(256), 0, st, a.proxy_map, s.n_b,
                       s.n_words, 0.f, 0, a.topk, 0.f, a.mask, a.kept, a.idx);
  else
    hipLaunchKernelGGL((route_select_kernel<kRouteTopP>), grid, dim3(256), 0, st, a.proxy_map, s.n_b,
                       s.n_words, 0.f, 0, 0, a.topp, a.mask, a.kept, a.idx);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Shape& s, Dtype dt, const RouteArgs& a, hipStream_t stream) {
  if (dt == Dtype::BF16)
    return s.d == 64 ? route_impl<__bf16, 64>(s, a, stream) : route_impl<__bf16, 128>(s, a, stream);
  return s.d == 64 ? route_impl<float, 64>(s, a, stream) : route_impl<float, 128>(s, a, stream);
}

}  // namespace sol
