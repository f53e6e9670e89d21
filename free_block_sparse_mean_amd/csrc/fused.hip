// Fused Sol-Attn forward pass for gfx950: threshold routing + exact sparse
// attention on bf16 MFMA + proxy-score-reuse correction, one online-softmax
// state per query row, nothing written to HBM but the output (and opt-in stats).
//
// Method sources (page "Sol-Attn: l'attenzione sparsa che sceglie al volo,
// per generare video piu in fretta", paithon.it):
//   section "Una soglia per ogni riga": tau_i = mu_i + beta*sigma_i with mu_i,
//     sigma_i in closed form from the key-summary mean m and d x d second
//     moments C; S_i = {j : s_hat_ij > tau_i};
//   section "Scegliere mentre si calcola": an outer loop over the compressed
//     keys produces the proxy scores and tests them against tau_i as they
//     appear; kept blocks go to an inner loop over the original K and V for
//     exact attention; excluded blocks are reused as zeroth-order terms (the
//     block-mean key for all its tokens) in the same softmax state.
//
// One workgroup (4 waves, 256 lanes) per query block i of one (b, h):
//   1. stage Q_i (64 x d) in LDS, q_bar_i by column sums, Q operands to VGPRs;
//   2. tau_i from q_bar_i, m and C (C read once from L2, 64 KiB at d = 128);
//   3. outer loop over key blocks: lane-per-block proxy scores from the
//      transposed summaries k_bar^T (coalesced rows of n_b floats); the strict
//      test against tau_i is folded into 64-bit wave ballots, one word per 64
//      key blocks, kept in LDS (never in HBM);
//   4. correction accumulators for the unselected blocks: own running max c_i,
//      weights w_j = exp(s_hat_ij - c_i), L_i = 64 sum w_j, A_i = sum w_j vsum_j;
//   5. inner loop over the set bits: K_j and V_j^T staged in LDS, per wave 16
//      query rows x 64 keys: S^T = K_j Q^T and O^T += V_j^T P^T with
//      v_mfma_f32_16x16x32_bf16, online softmax in base 2 in fp32, P as bf16;
//   6. epilogue: out = (O 2^(m-M) + A 2^(c-M)) / (l 2^(m-M) + L 2^(c-M)).
// Each lane owns one query row (lane % 16) of its wave and a quarter of the
// keys / head dims (lane / 16), so row statistics need only two xor-shuffles
// and rescaling is lane-local.
//
// Bound: bf16 MFMA on the kept tiles (4*64*64*d flop per kept block); the
// summary scan and the correction read n_b*d*4 bytes each per query block
// from L2.
//
// The float32 instantiation (small problems, tighter tolerance) keeps the same
// routing and correction and replaces step 5 by fp32 VALU dot products.
#include <type_traits>

#include "device_common.hpp"
#include "sol_internal.hpp"

namespace sol {
namespace {

struct FusedParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* kbar_t;
  const float* vsum;
  const float* kmean;
  const float* kcov;
  int n_b, n_b_pad, n_words;
  long long N;
  float beta;
  int beta_mode;
  int32_t* kept_per_row;
  uint64_t* mask_bits;
  float* tau_out;
};

template <typename T, int D> struct Geom;
template <int D> struct Geom<__bf16, D> {
  static constexpr int kKPitch = D + 8;     // elements per K (and staged Q) row
  static constexpr int kVPitch = 64 + 8;    // elements per V^T row
  static constexpr int kKBytes = 64 * kKPitch * 2;
  static constexpr int kVBytes = D * kVPitch * 2;
};
template <int D> struct Geom<float, D> {
  static constexpr int kKPitch = D + 4;
  static constexpr int kVPitch = D + 4;
  static constexpr int kKBytes = 64 * kKPitch * 4;
  static constexpr int kVBytes = 64 * kVPitch * 4;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

template <typename T, int D> struct Lds {
  static constexpr int kStage = Geom<T, D>::kKBytes + Geom<T, D>::kVBytes;
  __host__ __device__ static int sh(int) { return kStage; }
  __host__ __device__ static int masks(int n_b) { return kStage + align16(4 * n_b); }
  __host__ __device__ static int qbar(int n_b) {
    return masks(n_b) + align16(8 * ((n_b + 63) / 64));
  }
  __host__ __device__ static int acc(int n_b) { return qbar(n_b) + 4 * D; }
  __host__ __device__ static int misc(int n_b) { return acc(n_b) + 4 * 256; }
  __host__ __device__ static int bytes(int n_b) { return misc(n_b) + 4 * 16; }
};

constexpr float inv_sqrt(int d) { return d == 64 ? 0.125f : 0.08838834764831845f; }

// Sum over the workgroup of one float per thread; every thread gets the total.
__device__ inline float block_sum(float x, float* red) {
  x = wave_sum(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}
__device__ inline float block_max(float x, float* red) {
  x = wave_max(x);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <typename T, int D, bool CORR>
__global__ __launch_bounds__(256) void fused_kernel(FusedParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  using G = Geom<T, D>;
  using L = Lds<T, D>;
  constexpr float kInvSqrtD = inv_sqrt(D);
  constexpr float kScale2 = kInvSqrtD * kLog2e;   // logit -> base-2 exponent

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n_b = p.n_b;
  const long long item = blockIdx.x;
  const long long bh = item / n_b;
  const int qi = (int)(item - bh * n_b);

  T* stK = reinterpret_cast<T*>(lds);
  T* stV = reinterpret_cast<T*>(lds + G::kKBytes);
  float* sh = reinterpret_cast<float*>(lds + L::sh(n_b));
  uint64_t* masks = reinterpret_cast<uint64_t*>(lds + L::masks(n_b));
  float* qbar = reinterpret_cast<float*>(lds + L::qbar(n_b));
  float* accbuf = reinterpret_cast<float*>(lds + L::acc(n_b));
  float* misc = reinterpret_cast<float*>(lds + L::misc(n_b));

  const T* Qg = static_cast<const T*>(p.q) + ((size_t)bh * p.N + (size_t)qi * kBlock) * D;
  const T* Kg = static_cast<const T*>(p.k) + (size_t)bh * p.N * D;
  const T* Vg = static_cast<const T*>(p.v) + (size_t)bh * p.N * D;

  // ---- 1. Q tile -> LDS (K slot), q_bar, Q operands -------------------------
  {
    using V16 = Vec16<T>;
    constexpr int E = V16::kN, CH = D / E;
    for (int c = t; c < 64 * CH; c += 256) {
      const int r = c / CH, cc = c % CH;
      *reinterpret_cast<typename V16::raw*>(stK + r * G::kKPitch + cc * E) =
          reinterpret_cast<const typename V16::raw*>(Qg + (size_t)r * D)[cc];
    }
  }
  __syncthreads();
  {
    constexpr int P = 256 / D;
    const int c = t % D, part = t / D;
    float s = 0.f;
    for (int r = part; r < 64; r += P) s += (float)stK[r * G::kKPitch + c];
    accbuf[t] = s;
  }
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll
    for (int part = 0; part < 256 / D; ++part) s += accbuf[part * D + t];
    qbar[t] = s * (1.0f / kBlock);
  }
  const int row = 16 * w + (lane & 15);   // this lane's query row within the block
  const int grp = lane >> 4;              // this lane's quarter of keys / dims
  constexpr int KS = D / 32;
  bf16x8 qop[std::is_same<T, __bf16>::value ? KS : 1];
  float qf[std::is_same<T, float>::value ? D / 4 : 1];
  if constexpr (std::is_same<T, __bf16>::value) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = *reinterpret_cast<const bf16x8*>(stK + row * G::kKPitch + ks * 32 + grp * 8);
  } else {
#pragma unroll
    for (int e = 0; e < D / 4; ++e) qf[e] = stK[row * G::kKPitch + grp * (D / 4) + e];
  }
  __syncthreads();

  // ---- 2. threshold tau_i = mu_i + beta sigma_i (closed form) ---------------
  float tau;
  {
    const float* C = p.kcov + (size_t)bh * D * D;
    const float* m = p.kmean + (size_t)bh * D;
    constexpr int P = 256 / D;
    const int r = t % D, part = t / D;
    float y = 0.f;
    for (int c = part; c < D; c += P) y += C[(size_t)c * D + r] * qbar[c];
    const float qcq = block_sum(qbar[r] * y, misc);
    const float qm = block_sum(t < D ? qbar[t] * m[t] : 0.f, misc + 4);
    const float mu = qm * kInvSqrtD;
    const float sigma = sqrtf(fmaxf(qcq, 0.f) * (1.0f / D));
    if (p.beta_mode == kBetaMinusInf) tau = -INFINITY;
    else if (p.beta_mode == kBetaPlusInf) tau = INFINITY;
    else tau = mu + p.beta * sigma;
  }

  // ---- 3a. outer loop: proxy scores of every key block ----------------------
  {
    const float* kt = p.kbar_t + (size_t)bh * D * p.n_b_pad;
    for (int j4 = 4 * t; j4 < n_b; j4 += 1024) {
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll 16
      for (int c = 0; c < D; ++c) {
        const float4 kv = *reinterpret_cast<const float4*>(kt + (size_t)c * p.n_b_pad + j4);
        const float qc = qbar[c];
        a0 += qc * kv.x; a1 += qc * kv.y; a2 += qc * kv.z; a3 += qc * kv.w;
      }
      sh[j4] = a0 * kInvSqrtD;
      if (j4 + 1 < n_b) sh[j4 + 1] = a1 * kInvSqrtD;
      if (j4 + 2 < n_b) sh[j4 + 2] = a2 * kInvSqrtD;
      if (j4 + 3 < n_b) sh[j4 + 3] = a3 * kInvSqrtD;
    }
  }
  __syncthreads();

  // ---- 3b. strict test against tau_i -> one 64-bit word per 64 key blocks ---
  float cmax = -INFINITY;
  int kept = 0;
  for (int g = w; g < p.n_words; g += 4) {
    const int j = g * 64 + lane;
    const bool valid = j < n_b;
    const float s = valid ? sh[j] : 0.f;
    const bool keep = valid && (s > tau);
    const uint64_t word = __ballot(keep);
    if (valid && !keep) cmax = fmaxf(cmax, s);
    if (lane == 0) masks[g] = word;
    kept += __popcll(word);
  }
  cmax = block_max(cmax, misc);
  {
    __syncthreads();
    if (lane == 0) misc[8 + w] = (float)kept;
    __syncthreads();
    kept = (int)(misc[8] + misc[9] + misc[10] + misc[11]);
  }
  const long long qrow = bh * n_b + qi;
  if (t == 0) {
    if (p.kept_per_row) p.kept_per_row[qrow] = kept;
    if (p.tau_out) p.tau_out[qrow] = tau;
  }
  if (p.mask_bits)
    for (int g = t; g < p.n_words; g += 256) p.mask_bits[qrow * p.n_words + g] = masks[g];

  // ---- 4. correction: unselected blocks as 64 virtual tokens ---------------
  float c2 = -INFINITY, Lsum = 0.f;
  if constexpr (CORR) {
    if (cmax > -INFINITY) {
      c2 = cmax * kLog2e;
      float part_l = 0.f;
      for (int j = t; j < n_b; j += 256) {
        const bool keep = (masks[j >> 6] >> (j & 63)) & 1ull;
        const float wj = keep ? 0.f : exp2f(sh[j] * kLog2e - c2);
        sh[j] = wj;
        part_l += wj;
      }
      Lsum = block_sum(part_l, misc) * (float)kBlock;   // syncs: sh is complete
      constexpr int P = 256 / D;
      const int col = t % D, part = t / D;
      const float* vs = p.vsum + (size_t)bh * n_b * D + col;
      float a = 0.f;
#pragma unroll 4
      for (int j = part; j < n_b; j += P) {
        const float wj = sh[j];
        if (wj != 0.f) a += wj * vs[(size_t)j * D];
      }
      accbuf[t] = a;
    }
  }
  __syncthreads();
  if constexpr (CORR) {
    if (c2 > -INFINITY && t < D) {
      float s = 0.f;
#pragma unroll
      for (int part = 0; part < 256 / D; ++part) s += accbuf[part * D + t];
      qbar[t] = s;   // q_bar is no longer needed: it now holds A_i
    }
  }

  // ---- 5. inner loop: exact attention on the kept blocks -------------------
  float mrow = -INFINITY, lrow = 0.f;
  constexpr int NACC = std::is_same<T, __bf16>::value ? D / 16 : 1;
  f32x4 oacc[NACC];
  float of[std::is_same<T, float>::value ? D / 4 : 1];
#pragma unroll
  for (int i = 0; i < NACC; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (int)(sizeof(of) / sizeof(float)); ++i) of[i] = 0.f;

  for (int g = 0; g < p.n_words; ++g) {
    uint64_t word = masks[g];
    while (word) {
      const int j = g * 64 + (int)__builtin_ctzll(word);
      word &= word - 1;
      const T* Kj = Kg + (size_t)j * kBlock * D;
      const T* Vj = Vg + (size_t)j * kBlock * D;
      __syncthreads();   // previous tile fully consumed
      if constexpr (std::is_same<T, __bf16>::value) {
        // K_j natural [key][d]
        constexpr int CH = D / 8;
#pragma unroll
        for (int c = t; c < 64 * CH; c += 256) {
          const int r = c / CH, cc = c % CH;
          *reinterpret_cast<uint4*>(stK + r * G::kKPitch + cc * 8) =
              reinterpret_cast<const uint4*>(Kj + (size_t)r * D)[cc];
        }
        // V_j transposed [d][key]: lane takes KPT keys x 8 dims
        constexpr int KPT = D / 32;          // 4 at d = 128, 2 at d = 64
        const int dc = t % CH, kg = t / CH;  // kg in [0, 64 / KPT)
        uint4 raw[KPT];
#pragma unroll
        for (int r = 0; r < KPT; ++r)
          raw[r] = reinterpret_cast<const uint4*>(Vj + (size_t)(kg * KPT + r) * D)[dc];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          unsigned short h[KPT];
#pragma unroll
          for (int r = 0; r < KPT; ++r) {
            const uint32_t word32 = (&raw[r].x)[e >> 1];
            h[r] = (unsigned short)((e & 1) ? (word32 >> 16) : (word32 & 0xffffu));
          }
          T* dst = stV + (dc * 8 + e) * G::kVPitch + kg * KPT;
          if constexpr (KPT == 4) {
            *reinterpret_cast<uint2*>(dst) =
                make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
          } else {
            *reinterpret_cast<uint32_t*>(dst) = h[0] | ((uint32_t)h[1] << 16);
          }
        }
      } else {
        constexpr int CH = D / 4;
        for (int c = t; c < 64 * CH; c += 256) {
          const int r = c / CH, cc = c % CH;
          *reinterpret_cast<float4*>(stK + r * G::kKPitch + cc * 4) =
              reinterpret_cast<const float4*>(Kj + (size_t)r * D)[cc];
          *reinterpret_cast<float4*>(stV + r * G::kVPitch + cc * 4) =
              reinterpret_cast<const float4*>(Vj + (size_t)r * D)[cc];
        }
      }
      __syncthreads();

      if constexpr (std::is_same<T, __bf16>::value) {
        // S^T (64 keys x 16 queries of this wave): 4 key tiles of 16
        f32x4 s[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                stK + (kt * 16 + (lane & 15)) * G::kKPitch + ks * 32 + grp * 8);
            s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[ks], s[kt], 0, 0, 0);
          }
        }
        // online softmax (base 2): lane holds keys kt*16 + grp*4 + i of query `row`
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[kt][i]);
        tmax *= kScale2;
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mnew = fmaxf(mrow, tmax);
        const float alpha = exp2f(mrow - mnew);
        float psum = 0.f;
        bf16x8 pop[2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = exp2f(s[kt][i] * kScale2 - mnew);
            psum += pv;
            pop[kt >> 1][(kt & 1) * 4 + i] = to_bf16(pv);
          }
        lrow = lrow * alpha + psum;
        mrow = mnew;
#pragma unroll
        for (int dt = 0; dt < NACC; ++dt) oacc[dt] *= alpha;
        // O^T (d x 16 queries) += V^T (d x 64 keys) P^T: two k-steps of 32 keys
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int dt = 0; dt < NACC; ++dt) {
            const T* src = stV + (dt * 16 + (lane & 15)) * G::kVPitch + ks * 32 + grp * 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(src);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(src + 16);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop[ks], oacc[dt], 0, 0, 0);
          }
        }
      } else {
        // fp32: 4 lanes per query row, each a quarter of the head dims
        float sv[64];
        float tmax = -INFINITY;
#pragma unroll
        for (int key = 0; key < 64; ++key) {
          const float* kr = stK + key * G::kKPitch + grp * (D / 4);
          float a = 0.f;
#pragma unroll
          for (int e = 0; e < D / 4; ++e) a += qf[e] * kr[e];
          a += __shfl_xor(a, 16, 64);
          a += __shfl_xor(a, 32, 64);
          sv[key] = a * kScale2;
          tmax = fmaxf(tmax, sv[key]);
        }
        const float mnew = fmaxf(mrow, tmax);
        const float alpha = exp2f(mrow - mnew);
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < D / 4; ++e) of[e] *= alpha;
#pragma unroll
        for (int key = 0; key < 64; ++key) {
          const float pv = exp2f(sv[key] - mnew);
          psum += pv;
          const float* vr = stV + key * G::kVPitch + grp * (D / 4);
#pragma unroll
          for (int e = 0; e < D / 4; ++e) of[e] += pv * vr[e];
        }
        lrow = lrow * alpha + psum;
        mrow = mnew;
      }
    }
  }

  // ---- 6. epilogue: merge exact and virtual terms, normalise ---------------
  if constexpr (std::is_same<T, __bf16>::value) {
    lrow += __shfl_xor(lrow, 16, 64);   // lanes of one row held partial key sums
    lrow += __shfl_xor(lrow, 32, 64);
  }
  __syncthreads();   // A_i in qbar[] is visible
  const float M = fmaxf(mrow, c2);
  const float fo = (mrow == -INFINITY) ? 0.f : exp2f(mrow - M);
  const float fc = (c2 == -INFINITY) ? 0.f : exp2f(c2 - M);
  const float den = lrow * fo + Lsum * fc;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  T* orow = static_cast<T*>(p.out) + ((size_t)bh * p.N + (size_t)qi * kBlock + row) * D;
  if constexpr (std::is_same<T, __bf16>::value) {
#pragma unroll
    for (int dt = 0; dt < NACC; ++dt) {
      const int d0 = dt * 16 + grp * 4;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (c2 > -INFINITY) ? qbar[d0 + i] * fc : 0.f;
        o[i] = (oacc[dt][i] * fo + a) * inv;
      }
      bf16x4 ob = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
      *reinterpret_cast<bf16x4*>(orow + d0) = ob;
    }
  } else {
#pragma unroll
    for (int e = 0; e < D / 4; e += 4) {
      const int d0 = grp * (D / 4) + e;
      float4 o;
      float* op = &o.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (c2 > -INFINITY) ? qbar[d0 + i] * fc : 0.f;
        op[i] = (of[e + i] * fo + a) * inv;
      }
      *reinterpret_cast<float4*>(orow + d0) = o;
    }
  }
}

template <typename T, int D>
hipError_t fused_impl(const Shape& s, const FusedArgs& a, hipStream_t st) {
  FusedParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.out = a.out;
  p.kbar_t = a.ws.kbar_t; p.vsum = a.ws.vsum; p.kmean = a.ws.kmean; p.kcov = a.ws.kcov;
  p.n_b = s.n_b; p.n_b_pad = s.n_b_pad; p.n_words = s.n_words; p.N = s.N;
  p.beta = a.beta; p.beta_mode = a.beta_mode;
  p.kept_per_row = a.kept_per_row; p.mask_bits = a.mask_bits; p.tau_out = a.tau;
  const int lds = Lds<T, D>::bytes(s.n_b);
  const dim3 grid((unsigned)(s.BH() * s.n_b));
  if (a.correction) {
    auto k = fused_kernel<T, D, true>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, dim3(256), lds, st, p);
  } else {
    auto k = fused_kernel<T, D, false>;
    hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, dim3(256), lds, st, p);
  }
  return hipGetLastError();
}

}  // namespace

int fused_lds_bytes(Dtype dt, int d, int n_b) {
  if (dt == Dtype::BF16) return d == 64 ? Lds<__bf16, 64>::bytes(n_b) : Lds<__bf16, 128>::bytes(n_b);
  return d == 64 ? Lds<float, 64>::bytes(n_b) : Lds<float, 128>::bytes(n_b);
}

hipError_t launch_fused(const Shape& s, Dtype dt, const FusedArgs& a, hipStream_t stream) {
  if (dt == Dtype::BF16)
    return s.d == 64 ? fused_impl<__bf16, 64>(s, a, stream) : fused_impl<__bf16, 128>(s, a, stream);
  return s.d == 64 ? fused_impl<float, 64>(s, a, stream) : fused_impl<float, 128>(s, a, stream);
}

}  // namespace sol
