// Internal interface between the C-ABI host runtime (api.cpp) and the HIP
// kernels (prepass.hip, fused.hip). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sol {

constexpr int kBlock = 64;          // tokens per block
constexpr int kMaxBlocks = 4096;    // n_b limit (N <= 262144), bounded by the fused kernel's LDS
constexpr int kCovChunk = 128;      // key blocks per covariance partial (halved to 32 for small problems)

enum class Dtype { BF16, F32 };

// beta handling without forming beta * sigma for infinite beta
enum BetaMode : int { kBetaFinite = 0, kBetaMinusInf = 1, kBetaPlusInf = 2 };

struct Shape {
  int B, H, N, d;
  int n_b;      // N / 64
  int n_b_pad;  // n_b rounded up to a multiple of 4 (row pitch of kbar_t)
  int n_words;  // ceil(n_b / 64): mask words per query block
  int cov_chunk;  // key blocks per covariance partial: kCovChunk, 64 or 32 (small problems)
  int cov_parts;  // ceil(n_b / cov_chunk)
  long long BH() const { return (long long)B * H; }
};

// Element strides of one [B][H][N][d] tensor whose rows of d values are
// contiguous: element (ib, ih, t, c) sits at ib*b + ih*h + t*n + c. The default
// (contiguous BHND) is {H*N*d, N*d, d}; BNHD is {N*H*d, d, H*d}.
struct TStrides {
  long long b, h, n;
};
inline TStrides contiguous_strides(const Shape& s) {
  return TStrides{(long long)s.H * s.N * s.d, (long long)s.N * s.d, (long long)s.d};
}
struct IoStrides {
  TStrides q, k, v, o;
};
inline IoStrides contiguous_io(const Shape& s) {
  const TStrides c = contiguous_strides(s);
  return IoStrides{c, c, c, c};
}

struct Workspace {
  float* kbar_t;    // [BH][d][n_b_pad]
  float* kbar;      // [BH][n_b][d]
  float* vsum;      // [BH][n_b][d]
  float* kmean;     // [BH][d]
  float* kcov;      // [BH][d][d]
  __bf16* vt;       // [BH][n_b][d][64]  V blocks transposed (bf16 inputs only)
  float* qbar;      // [BH][n_b][d]      block-mean queries (routing baselines only)
  __bf16* kbar_bf;  // [BH][n_words][64][d]  k_bar as bf16 tiles (per-row correction; bf16 only)
  __bf16* vbar_t;   // [BH][n_words][d][64]  v_bar as bf16 V^T-order tiles (per-row correction)
  __bf16* vbar_bf;  // [BH][n_words][64][d]  v_bar as bf16 row-major tiles (per-row correction, low memory)
  double* s1_part;  // [BH][cov_parts][d]     (pre-pass scratch)
  double* s2_part;  // [BH][cov_parts][d][d]  (pre-pass scratch)
};

struct Layout {
  // vt is the last array: the workspace of the low-memory mode (no V^T copy)
  // is the first `vt` bytes of the full one
  size_t kbar_t, kbar, vsum, kmean, kcov, qbar, kbar_bf, vbar_t, vbar_bf, s1_part, s2_part, vt, total;
};

Layout make_layout(const Shape& s);
Workspace bind_workspace(const Shape& s, void* base);

// Launch geometry of the fused pass (shared by the host runtime and tests).
struct FusedGeom {
  int G;            // query blocks per workgroup
  int n_groups;     // ceil(n_b / G) per head
  long long items;  // BH * n_groups
  long long per_xcd;  // ceil(n_groups / 8): work items of one head per XCD
  int dyn_heads;      // trailing heads whose work items are dealt from a queue
  long long n_static_wg;  // workgroups of the statically mapped heads
  long long workers;      // queue workers (twice the queued items, at most one item each)
  int lds_bytes;
};
FusedGeom fused_geom(const Shape& s, Dtype dt);

struct FusedArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  Workspace ws;
  float beta;
  int beta_mode;
  bool correction;
  bool correction_row;   // per-row correction logit q_r . k_bar_j (instead of s_hat_ij)
  int32_t* kept_per_row;
  uint64_t* mask_bits;
  float* tau;
  uint64_t* item_clock;
  const uint64_t* mask_in;   // non-null: caller-given selection, no routing and no correction
  int text_blocks;           // joint attention: the last text_blocks blocks are text (always exact)
  IoStrides io;              // element strides of q, k, v and out
  bool low_memory;           // bf16: V tiles from the input V (transposing LDS reads), no V^T copy
};

// Routing baselines with a materialized proxy map (route.hip).
enum RouteMode : int { kRouteThreshold = 0, kRouteTopK = 1, kRouteTopP = 2 };
struct RouteArgs {
  const void* q;
  TStrides qs;         // element strides of q
  Workspace ws;        // pre-pass summaries of K (kbar) and room for qbar
  int mode;
  float beta;
  int beta_mode;
  int topk;
  float topp;
  float* proxy_map;    // [BH][n_b][n_b]
  uint64_t* mask;      // [BH][n_b][n_words]
  int32_t* kept;       // [BH][n_b] or null
  int32_t* idx;        // [BH][n_b][topk] or null (top-k only)
};

// Each returns the first HIP error of its launches (hipSuccess otherwise).
// write_vt: write the bf16 V^T copy (not in the low-memory mode)
hipError_t launch_prepass(const Shape& s, Dtype dt, const void* k, const void* v, const TStrides& ks,
                          const TStrides& vs, const Workspace& ws, bool write_vt, hipStream_t stream);
hipError_t launch_fused(const Shape& s, Dtype dt, const FusedArgs& a, hipStream_t stream);
// The bf16 per-row-correction fused kernel for head dim d (64 or 128), compiled
// in a translation unit of its own (fused.hip with SOL_FUSED_ROW_TU).
const void* fused_row_kernel_bf16(int d, bool low_memory);
// That translation unit's queue-slot reset kernel (its own slot pool).
const void* fused_row_reset_kernel();
hipError_t launch_route(const Shape& s, Dtype dt, const RouteArgs& a, hipStream_t stream);

// Size of the static per-device scratch of sol_attn_fwd_noalloc (noalloc.hip).
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
// Device address of that scratch on the current device (looked up on the
// device's first call, then cached).
hipError_t noalloc_scratch(void** out);


}  // namespace sol
