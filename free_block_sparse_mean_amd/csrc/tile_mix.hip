// Issue-rate microbenchmark for the instruction mix of the fused pass's tile
// loop on gfx950: per step of 16 v_mfma_f32_16x16x32_bf16 (four accumulator
// chains, as S^T = K Q^T and O^T += V^T P^T issue them), a given number of
// 16-byte LDS operand reads (each feeding the MFMAs that follow it), FMAs and
// v_exp_f32. One workgroup per CU holds 1 or 2 waves per SIMD; the host times
// the launch with HIP events (the MFMA rate follows from the MFMA count).
//
// It measures what the hardware can issue, not the fused kernel: here the
// VALU work does not wait for MFMA results (in the tile loop the softmax
// waits for S), so each mix gives an upper bound for the loop of that shape.
// Not part of the attention library (its own shared object, libsoltilemix.so).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufVec = 512;          // 8 KB of bf16x8 operands in LDS
constexpr int kHogVec = 5 * 1024;     // 80 KB more LDS: at most one workgroup per CU

// NLDS operand reads, NVALU FMAs and NEXP exponentials per 16 MFMAs
template <int NLDS, int NVALU, int NEXP>
__global__ __launch_bounds__(512) void tile_mix_kernel(int iters, float* __restrict__ sink) {
  static_assert(NLDS == 0 || 16 % NLDS == 0, "operand reads must divide the 16 MFMAs evenly");
  // one array, operands first: their addresses stay within the 16-bit
  // immediate offset of the LDS reads
  __shared__ bf16x8 lds[kBufVec + kHogVec];
  bf16x8* buf = lds;
  const int t = threadIdx.x, lane = t & 63;
  for (int e = t; e < kBufVec; e += blockDim.x) {
    bf16x8 x;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (__bf16)(1e-3f * (float)((e + i) & 15));
    buf[e] = x;
  }
  lds[kBufVec + t][0] = (__bf16)(float)t;   // the reservation stays live
  __syncthreads();
  bf16x8 a = buf[lane];
  const bf16x8 b = buf[(lane + 64) & (kBufVec - 1)];
  f32x4 acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float v[8], x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[i] = 1.0f + 1e-3f * (float)(t + i);
    x[i] = 0.5f + 1e-4f * (float)(t + i);
  }
  for (int it = 0; it < iters; ++it) {
    // one address per step, the reads at constant offsets from it (as the
    // tile loop's operand reads): index at most 255 + 240 < kBufVec
    const bf16x8* p = buf + ((lane + it) & 255);
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      if constexpr (NLDS > 0) {
        if (m % (16 / NLDS) == 0) a = p[16 * m];   // a distinct address per read
      }
      acc[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[m & 3], 0, 0, 0);
      // this MFMA's share of the VALU work: FMAs and exponentials on
      // independent chains that stay bounded (fixed point 1, range [0.5, 1))
#pragma unroll
      for (int i = (m * NVALU) / 16; i < ((m + 1) * NVALU) / 16; ++i) v[i & 7] = fmaf(v[i & 7], 0.999f, 1e-3f);
#pragma unroll
      for (int i = (m * NEXP) / 16; i < ((m + 1) * NEXP) / 16; ++i) x[i & 7] = __builtin_amdgcn_exp2f(-x[i & 7]);
    }
  }
  float s = (float)lds[kBufVec + (t + 1) % blockDim.x][0];
#pragma unroll
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i] + x[i];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

// the mixes: pure MFMA; operand reads only; the softmax VALU work only; the
// tile loop's mix (one read per MFMA); half and a quarter of its reads
constexpr int kMixes = 6;
const void* mix_kernel(int mix) {
  switch (mix) {
    case 0: return (const void*)tile_mix_kernel<0, 0, 0>;
    case 1: return (const void*)tile_mix_kernel<16, 0, 0>;
    case 2: return (const void*)tile_mix_kernel<0, 24, 8>;
    case 3: return (const void*)tile_mix_kernel<16, 24, 8>;
    case 4: return (const void*)tile_mix_kernel<8, 24, 8>;
    case 5: return (const void*)tile_mix_kernel<4, 24, 8>;
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

// Describes mix `mix`: operand reads, FMAs and exponentials per 16 MFMAs.
// Returns 0, or -1 for an unknown mix.
int sol_tile_mix_shape(int mix, int* lds_reads, int* fmas, int* exps) {
  static const int shape[kMixes][3] = {{0, 0, 0}, {16, 0, 0}, {0, 24, 8}, {16, 24, 8}, {8, 24, 8}, {4, 24, 8}};
  if (mix < 0 || mix >= kMixes || !lds_reads || !fmas || !exps) return -1;
  *lds_reads = shape[mix][0];
  *fmas = shape[mix][1];
  *exps = shape[mix][2];
  return 0;
}

// Runs mix `mix` with `waves_per_simd` (1 or 2) waves on every SIMD of the
// current device (one workgroup per CU), `iters` steps of 16 MFMAs per wave,
// once untimed and once timed with HIP events on the null stream; writes the
// timed launch's milliseconds to *ms and the CU count to *cus_out. Allocates
// and frees its own device buffer. Returns 0 or a HIP error code (-1 for bad
// arguments, checked before any device call).
int sol_tile_mix(int mix, int waves_per_simd, int iters, double* ms, int* cus_out) {
  if (!mix_kernel(mix) || (waves_per_simd != 1 && waves_per_simd != 2) || iters < 1 || iters > (1 << 24) || !ms ||
      !cus_out)
    return -1;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  const int threads = 256 * waves_per_simd;
  float* sink = nullptr;
  if ((e = hipMalloc(&sink, sizeof(float) * (size_t)cus * threads)) != hipSuccess) return (int)e;
  hipEvent_t ev[2] = {nullptr, nullptr};
  e = hipEventCreate(&ev[0]);
  if (e == hipSuccess) e = hipEventCreate(&ev[1]);
  void* args[] = {&iters, &sink};
  if (e == hipSuccess) e = hipLaunchKernel(mix_kernel(mix), dim3(cus), dim3(threads), args, 0, nullptr);
  if (e == hipSuccess) e = hipEventRecord(ev[0], nullptr);
  if (e == hipSuccess) e = hipLaunchKernel(mix_kernel(mix), dim3(cus), dim3(threads), args, 0, nullptr);
  if (e == hipSuccess) e = hipEventRecord(ev[1], nullptr);
  if (e == hipSuccess) e = hipEventSynchronize(ev[1]);
  float t = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&t, ev[0], ev[1]);
  for (hipEvent_t x : ev)
    if (x) (void)hipEventDestroy(x);
  (void)hipFree(sink);
  if (e != hipSuccess) return (int)e;
  *ms = t;
  *cus_out = cus;
  return 0;
}

}  // extern "C"
