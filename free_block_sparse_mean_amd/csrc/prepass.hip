// Block-summary pre-pass for Sol-Attn on gfx950.
//
// Reads K and V once and produces what the fused pass needs to route every
// query block without forming a row of proxy scores:
//   k_bar_j = mean of the 64 keys of block j         (row-major and transposed)
//   vsum_j  = sum of the 64 values of block j        (= 64 * v_bar_j)
//   m       = mean over j of k_bar_j
//   C       = (1/n_b) sum_j k_bar_j k_bar_j^T - m m^T   (population covariance)
// and, for bf16 inputs, a copy of V with every 64 x d block transposed to
// d x 64, keys permuted within each group of 32 into the order the fused
// pass feeds them to its P.V MFMA (one 16-byte LDS read per operand).
// Sources: page "Sol-Attn: l'attenzione sparsa che sceglie al volo"
// (paithon.it), section "Perche l'attenzione pesa tanto nei video" for the
// 64-token block means, section "Una soglia per ogni riga" (last paragraph)
// for mu_i/sigma_i from the mean of the compressed keys and their d x d
// second-moment matrix, and section "Scegliere mentre si calcola" for the
// block-mean values the correction reuses.
//
// Bound: HBM bandwidth. block_sums streams 2*N*d input elements per head
// with 16-byte loads, one wave per block (and writes N*d transposed values
// for bf16). The moment kernels touch only the n_b x d summaries
// (L2-resident) and accumulate in double, so forming C from second moments
// loses nothing to cancellation at fp32 resolution.
#include <type_traits>

#include "device_common.hpp"
#include "sol_internal.hpp"

namespace sol {
namespace {

// Chunk swizzle of row r of a staged V block (CH 16-byte chunks per row): the
// transposing reads below gather keys k0 + c for the eight k0 of one output
// chunk row (4 apart within each half of 32 keys); this maps them to eight
// distinct chunk slots.
template <int CH>
__device__ __forceinline__ int vt_swz(int r) {
  return ((r >> 2) ^ ((r >> 5) << 2)) & (CH - 1);
}

// One wave per key block: lane (rg, cc) sums rows rg, rg+RG, ... of 16-byte
// column chunk cc for K and V, then the row groups are folded by xor-shuffles.
// With WRITE_VT the wave also stages its V block in LDS and writes it back
// transposed ([d][64] per block).
template <typename T, int D, bool WRITE_VT>
__global__ __launch_bounds__(256) void block_sums_kernel(const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         float* __restrict__ kbar,
                                                         float* __restrict__ vsum,
                                                         __bf16* __restrict__ vt,
                                                         int n_b, int H, TStrides ks, TStrides vs) {
  using V = Vec16<T>;
  constexpr int E = V::kN;     // elements per 16-byte chunk
  constexpr int CH = D / E;    // chunks per row
  constexpr int RG = 64 / CH;  // row groups
  constexpr int RPL = 64 / RG; // rows per lane
  constexpr int kPitch = D;    // unpadded: row writes are whole 16-byte chunks
  __shared__ __attribute__((aligned(16))) __bf16 stage[WRITE_VT ? 4 : 1][WRITE_VT ? 64 * kPitch : 8];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int j = blockIdx.x * 4 + wv;
  const long long bh = blockIdx.y;
  if (j >= n_b) return;   // whole wave leaves; no workgroup barrier below
  const int cc = lane % CH, rg = lane / CH;
  const long long ib = bh / H, ih = bh % H;
  const T* kb0 = k + ib * ks.b + ih * ks.h + (long long)j * kBlock * ks.n;   // row 0 of key block j
  const T* vb0 = v + ib * vs.b + ih * vs.h + (long long)j * kBlock * vs.n;
  float ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) { ak[e] = 0.f; av[e] = 0.f; }
  // every load of the block first (all 2 * RPL of them in flight: the LDS
  // stage caps a CU at eight waves, so each wave keeps its whole block moving)
  typename V::raw rkr[RPL], rvr[RPL];
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int r = rg + RG * i;
    rkr[i] = reinterpret_cast<const typename V::raw*>(kb0 + (long long)r * ks.n)[cc];
    rvr[i] = reinterpret_cast<const typename V::raw*>(vb0 + (long long)r * vs.n)[cc];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < RPL; ++i) {
    const int r = rg + RG * i;
    float fk[E], fv[E];
    V::to_float(rkr[i], fk);
    V::to_float(rvr[i], fv);
#pragma unroll
    for (int e = 0; e < E; ++e) { ak[e] += fk[e]; av[e] += fv[e]; }
    if constexpr (WRITE_VT)
      *reinterpret_cast<typename V::raw*>(&stage[wv][r * kPitch + (cc ^ vt_swz<CH>(r)) * E]) = rvr[i];
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
  if constexpr (WRITE_VT) {
    // The wave wrote the whole 64 x D block; LDS accesses of one wave are
    // performed in order, so a wave-level fence suffices before reading.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // Output chunk (d, kc) is 8 bf16 of head dim d: keys k0..k0+3 then
    // k0+16..k0+19 with k0 = 32*(kc/4) + 4*(kc%4), the order in which a lane
    // of the fused kernel holds P for one 16x16x32 MFMA k-step. Eight
    // consecutive lanes write the eight chunks of one d (128 contiguous
    // bytes), so each store covers 1 KB; the row swizzle of the staged block
    // puts the eight keys a read instruction gathers for one d in distinct
    // 16-byte slots (distinct LDS banks).
    __bf16* dst = vt + ((size_t)bh * n_b + j) * D * 64;
    for (int c = lane; c < D * 8; c += 64) {
      const int d = c >> 3, kc = c & 7;
      const int k0 = 32 * (kc >> 2) + 4 * (kc & 3);
      uint32_t w[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int ka = k0 + (h >> 1) * 16 + 2 * (h & 1);
        const uint32_t lo = __builtin_bit_cast(
            unsigned short, stage[wv][ka * kPitch + ((d / E) ^ vt_swz<CH>(ka)) * E + (d % E)]);
        const uint32_t hi = __builtin_bit_cast(
            unsigned short, stage[wv][(ka + 1) * kPitch + ((d / E) ^ vt_swz<CH>(ka + 1)) * E + (d % E)]);
        w[h] = lo | (hi << 16);
      }
      *reinterpret_cast<uint4*>(dst + (size_t)d * 64 + kc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// Partial first and second moments of the key summaries over one chunk of
// `chunk` blocks (a multiple of 32), in double; also writes the transposed
// summaries kbar_t. One workgroup per (chunk, half z of the D x D partial):
// rows z*D/2 .. z*D/2 + D/2 - 1 and every column, as 16 x 16 tiles that the
// four waves share out (D = 128: wave w takes row tile w and all eight column
// tiles). The partial is X^T X over the chunk's rows X_j = k_bar_j; it runs
// on the fp64 MFMA (16x16x4: four key blocks per step), whose products of
// float-valued doubles are exact, with operands read from the staged tile
// (converted to double once).
template <int D>
__device__ __forceinline__ void moments_partial_body(const float* __restrict__ kbar,
                                                     float* __restrict__ kbar_t,
                                                     double* __restrict__ s1_part,
                                                     double* __restrict__ s2_part, int n_b, int n_b_pad,
                                                     int parts, int chunk, long long bh, int part, int z,
                                                     double* tile) {
  constexpr int TJ = 32;               // key blocks staged per step
  constexpr int kPitch = D + 1;        // doubles per staged row: the transposing reads hit distinct banks
  constexpr int CT = D / 16;           // column tiles
  constexpr int NT = (D / 32) * CT / 4;   // tiles per wave (half the row tiles x all column tiles, 4 waves)
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int i16 = lane & 15, kq = lane >> 4;   // MFMA operand lane: row/column i16 of key block kq
  const int j0 = part * chunk;
  const int j1 = min(n_b, j0 + chunk);
  const int r0 = z * (D / 2);
  f64x4 acc[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) acc[u] = f64x4{0.0, 0.0, 0.0, 0.0};
  double s1 = 0.0;

  // the next step's summaries are loaded into registers while the current
  // step is computed
  constexpr int NL = TJ * D / 256;   // staged values per thread
  float nxt[NL];
  auto fetch = [&](int jb) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = t + 256 * i, jj = e / D, c = e % D, j = jb + jj;
      nxt[i] = j < j1 ? kbar[((size_t)bh * n_b + j) * D + c] : 0.f;
    }
  };
  fetch(j0);
  for (int jb = j0; jb < j1; jb += TJ) {
    __syncthreads();   // every read of the previous step's tile is done
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = t + 256 * i;
      tile[(e / D) * kPitch + e % D] = (double)nxt[i];
    }
    __syncthreads();
    if (jb + TJ < j1) fetch(jb + TJ);
    // this half's columns of kbar_t (exact: the doubles came from floats)
    for (int e = t; e < TJ * (D / 2); e += 256) {
      const int c = r0 + e / TJ, jj = e % TJ, j = jb + jj;
      if (j < j1) kbar_t[((size_t)bh * D + c) * n_b_pad + j] = (float)tile[jj * kPitch + c];
    }
    if (z == 0 && t < D) {
      const int nj = min(TJ, j1 - jb);
      for (int jj = 0; jj < nj; ++jj) s1 += tile[jj * kPitch + t];
    }
    // rows past j1 were staged as zeros, so every step takes all TJ rows
#pragma unroll 2
    for (int jj = 0; jj < TJ; jj += 4) {
      const double* row = tile + (jj + kq) * kPitch;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int g = w * NT + u, rt = g / CT, ct = g % CT;
        acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(row[r0 + 16 * rt + i16], row[16 * ct + i16], acc[u], 0, 0, 0);
      }
    }
  }
  // zero this half's row padding of kbar_t once per head
  if (part == parts - 1) {
    const int pad = n_b_pad - n_b;
    for (int e = t; e < (D / 2) * pad; e += 256) {
      const int c = r0 + e / pad, j = n_b + e % pad;
      kbar_t[((size_t)bh * D + c) * n_b_pad + j] = 0.f;
    }
  }
  // the fp64 MFMA leaves row kq + 4 v of its tile, column i16, in item v of
  // a lane (unlike the fp32 16x16 forms, whose items are consecutive rows)
  double* outp = s2_part + ((size_t)bh * parts + part) * D * D;
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int g = w * NT + u, rt = g / CT, ct = g % CT;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      outp[(size_t)(r0 + 16 * rt + kq + 4 * v) * D + 16 * ct + i16] = acc[u][v];
  }
  if (z == 0 && t < D) s1_part[((size_t)bh * parts + part) * D + t] = s1;
}

// m = (sum of the S1 partials) / n_b and C = (sum of the S2 partials) / n_b - m m^T,
// partials summed in chunk order (deterministic), stored as float.
template <int D>
__global__ __launch_bounds__(256) void moments_reduce_kernel(const double* __restrict__ s1_part,
                                                             const double* __restrict__ s2_part,
                                                             float* __restrict__ kmean,
                                                             float* __restrict__ kcov, int n_b,
                                                             int parts) {
  __shared__ double m[D];
  const long long bh = blockIdx.y;
  const int t = threadIdx.x;
  if (t < D) {
    double s = 0.0;
    for (int p = 0; p < parts; ++p) s += s1_part[((size_t)bh * parts + p) * D + t];
    m[t] = s / (double)n_b;
    if (blockIdx.x == 0) kmean[(size_t)bh * D + t] = (float)m[t];
  }
  __syncthreads();
  const int e = blockIdx.x * 256 + t;
  if (e >= D * D) return;
  double s = 0.0;
  for (int p = 0; p < parts; ++p) s += s2_part[((size_t)bh * parts + p) * D * D + e];
  kcov[(size_t)bh * D * D + e] = (float)(s / (double)n_b - m[e / D] * m[e % D]);
}

// Block summaries as bf16 MFMA tiles, for the per-row correction: chunk c of
// 64 key blocks gives a K-like tile [64][D] of k_bar_j and a V^T-like tile
// [D][64] of v_bar_j = vsum_j / 64 in the column order of the V^T tiles; rows
// and columns past n_b are zero (the fused pass masks them out); and the same
// v_bar_j as a row-major [64][D] tile (write_rm: the low-memory mode's value tiles).
// One workgroup per (chunk c, quarter q of the head dims).
template <int D>
__device__ __forceinline__ void virtual_tiles_body(const float* __restrict__ kbar,
                                                   const float* __restrict__ vsum,
                                                   __bf16* __restrict__ kbar_bf,
                                                   __bf16* __restrict__ vbar_t,
                                                   __bf16* __restrict__ vbar_bf, int n_b,
                                                   int n_chunks, int write_rm, long long bh, int c,
                                                   int q) {
  constexpr int DQ = D / 4;   // head dims of this workgroup
  const int t = threadIdx.x, d0 = q * DQ;
  __bf16* kd = kbar_bf + ((size_t)bh * n_chunks + c) * 64 * D;
  __bf16* vr = vbar_bf + ((size_t)bh * n_chunks + c) * 64 * D;
  for (int e = t; e < 64 * DQ; e += 256) {
    const int r = e / DQ, dd = d0 + e % DQ, j = 64 * c + r;
    kd[r * D + dd] = j < n_b ? to_bf16(kbar[((size_t)bh * n_b + j) * D + dd]) : to_bf16(0.f);
    if (write_rm)
      vr[r * D + dd] = j < n_b ? to_bf16(vsum[((size_t)bh * n_b + j) * D + dd] * (1.0f / kBlock)) : to_bf16(0.f);
  }
  __bf16* vd = vbar_t + ((size_t)bh * n_chunks + c) * D * 64;
  for (int e = d0 * 64 + t; e < (d0 + DQ) * 64; e += 256) {
    const int dd = e / 64, col = e % 64, kc = col / 8, ee = col % 8;
    const int j = 64 * c + 32 * (kc >> 2) + 4 * (kc & 3) + 16 * (ee >> 2) + (ee & 3);
    vd[e] = j < n_b ? to_bf16(vsum[((size_t)bh * n_b + j) * D + dd] * (1.0f / kBlock)) : to_bf16(0.f);
  }
}

template <int D>
__global__ __launch_bounds__(256) void moments_partial_kernel(const float* __restrict__ kbar,
                                                              float* __restrict__ kbar_t,
                                                              double* __restrict__ s1_part,
                                                              double* __restrict__ s2_part, int n_b,
                                                              int n_b_pad, int parts, int chunk) {
  __shared__ double tile[32 * (D + 1)];
  moments_partial_body<D>(kbar, kbar_t, s1_part, s2_part, n_b, n_b_pad, parts, chunk, blockIdx.y, blockIdx.x,
                          blockIdx.z, tile);
}

// A launch of its own, without the moment kernel's LDS tile: these workgroups
// are latency bound and need occupancy (sharing the moment kernel's launch,
// and so its LDS footprint, made the pair slower than two launches).
template <int D>
__global__ __launch_bounds__(256) void virtual_tiles_kernel(const float* __restrict__ kbar,
                                                            const float* __restrict__ vsum,
                                                            __bf16* __restrict__ kbar_bf,
                                                            __bf16* __restrict__ vbar_t,
                                                            __bf16* __restrict__ vbar_bf, int n_b,
                                                            int n_words, int write_rm) {
  virtual_tiles_body<D>(kbar, vsum, kbar_bf, vbar_t, vbar_bf, n_b, n_words, write_rm, blockIdx.y, blockIdx.x,
                        blockIdx.z);
}

template <typename T, int D>
hipError_t prepass_impl(const Shape& s, const void* k, const void* v, const TStrides& ks, const TStrides& vs,
                        const Workspace& ws, bool write_vt, hipStream_t st) {
  const unsigned bh = (unsigned)s.BH();
  constexpr bool kVT = std::is_same<T, __bf16>::value;
  if (kVT && write_vt)
    hipLaunchKernelGGL((block_sums_kernel<T, D, kVT>), dim3((s.n_b + 3) / 4, bh), dim3(256), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), ws.kbar, ws.vsum, ws.vt,
                       s.n_b, s.H, ks, vs);
  else
    hipLaunchKernelGGL((block_sums_kernel<T, D, false>), dim3((s.n_b + 3) / 4, bh), dim3(256), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), ws.kbar, ws.vsum, ws.vt,
                       s.n_b, s.H, ks, vs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((moments_partial_kernel<D>), dim3(s.cov_parts, bh, 2), dim3(256), 0, st, ws.kbar,
                     ws.kbar_t, ws.s1_part, ws.s2_part, s.n_b, s.n_b_pad, s.cov_parts, s.cov_chunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (kVT) {   // fp32 inputs have no summary tiles
    hipLaunchKernelGGL((virtual_tiles_kernel<D>), dim3(s.n_words, bh, 4), dim3(256), 0, st, ws.kbar, ws.vsum,
                       ws.kbar_bf, ws.vbar_t, ws.vbar_bf, s.n_b, s.n_words, write_vt ? 0 : 1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((moments_reduce_kernel<D>), dim3((D * D + 255) / 256, bh), dim3(256), 0, st,
                     ws.s1_part, ws.s2_part, ws.kmean, ws.kcov, s.n_b, s.cov_parts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepass(const Shape& s, Dtype dt, const void* k, const void* v, const TStrides& ks,
                          const TStrides& vs, const Workspace& ws, bool write_vt, hipStream_t stream) {
  if (dt == Dtype::BF16)
    return s.d == 64 ? prepass_impl<__bf16, 64>(s, k, v, ks, vs, ws, write_vt, stream)
                     : prepass_impl<__bf16, 128>(s, k, v, ks, vs, ws, write_vt, stream);
  return s.d == 64 ? prepass_impl<float, 64>(s, k, v, ks, vs, ws, write_vt, stream)
                   : prepass_impl<float, 128>(s, k, v, ks, vs, ws, write_vt, stream);
}

}  // namespace sol
