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
//     block-mean key for all their tokens) in the same softmax state.
//
// One workgroup (4 waves, 256 lanes) takes G consecutive query blocks of one
// (b, h) (G <= 4, chosen so their proxy rows fit in LDS):
//   1. q_bar for the G blocks from 16-byte loads of Q (wave shuffles + LDS);
//   2. tau for the G blocks from q_bar, m and C (C read once from L2);
//   3. outer loop over key blocks: lane-per-4-blocks proxy scores from the
//      transposed summaries k_bar^T, each k_bar value loaded once for all G
//      query blocks; the strict test against tau folded into 64-bit wave
//      ballots, one word per 64 key blocks, kept in LDS (never in HBM);
//   4. correction for the unselected blocks of each query block: own running
//      max c, weights w_j = exp(s_hat_j - c), L = 64 sum w_j, A = sum w_j vsum_j;
//      for bf16 inputs the weights are rounded to bf16 and A runs on MFMA
//      against bf16 tiles of v_bar^T (fp32: each vsum row loaded once for all
//      G blocks);
//   5. inner loop over the union of the G blocks' kept sets, in ascending
//      key-block order: each union tile's K and transposed V are loaded once,
//      straight from global memory into LDS, and computed for every block
//      that keeps it; two LDS buffers, so the next union tile loads while the
//      current one is computed. Each wave holds 16 query rows of every block;
//      S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16, online
//      softmax in base 2 in fp32, P rounded to bf16;
//   6. per query block: out = (O 2^(m-M) + A 2^(c-M)) / (l 2^(m-M) + L 2^(c-M)).
// Each lane owns one query row (lane % 16) of its wave and a quarter of the
// keys / head dims (lane / 16): row statistics need two permlane swaps and
// the rescale is lane-local.
//
// Workgroups are mapped head-synchronously: all XCDs work on the same head at
// a time (its K and V^T stay in the shared Infinity Cache), each XCD on a
// contiguous run of its query groups (neighbouring query blocks, which keep
// largely the same key blocks, share that XCD's L2).
//
// Bound: bf16 MFMA on the kept tiles (4*64*64*d flop per kept block); the
// summary scan and the correction read n_b*d*4 bytes each per G query blocks.
//
// Compiled twice: the bf16 kernels of the per-row correction are built alone
// in a translation unit of their own (SOL_FUSED_ROW_TU) with another
// scheduler, every other kernel in the main one.
//
// The float32 instantiation (small problems, tighter tolerance) keeps the same
// routing and correction and computes the kept tiles with fp32 VALU dot
// products from LDS-staged K and V, without prefetch.
#include <atomic>
#include <type_traits>

#include "device_common.hpp"
#include "queue_slots.hpp"
#include "sol_internal.hpp"

namespace sol {
namespace {

constexpr int kGMax = 4;

struct FusedParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const __bf16* vt;
  const __bf16* kbar_bf;   // block-summary tiles for the per-row correction (bf16)
  const __bf16* vbar_t;
  const __bf16* vbar_bf;   // the same v_bar tiles row-major (per-row correction, low-memory mode)
  const float* kbar;       // block means (fp32 per-row correction)
  const float* kbar_t;
  const float* vsum;
  const float* kmean;
  const float* kcov;
  int n_b, n_b_pad, n_words, G, n_groups;
  long long BH, per_xcd;   // per_xcd: work items of one head given to each XCD
  long long n_static_wg;   // workgroups of the statically mapped heads; the rest are queue workers
  int dyn_heads;           // the last dyn_heads heads' work items form the queue
  int qslot;               // this launch's queue counter in kQueue (zeroed before it)
  long long N;
  int H;
  TStrides qs, ks, vs, os;   // element strides of q, k, v and out (rows of d are contiguous)
  float beta;
  int beta_mode;
  int32_t* kept_per_row;
  uint64_t* mask_bits;
  float* tau_out;
  uint64_t* item_clock;
  const uint64_t* mask_in;   // caller-given selection (kModeGiven), [BH][n_b][n_words]
  int text_blocks;           // the last text_blocks blocks are text: always kept, dense rows
};

// Work-item queue counters, one per launch in flight (slots handed out by the
// host's QueueSlots pool, each zeroed by queue_reset_kernel on the launch's
// stream just before the launch): static device memory, nothing is allocated,
// and the workspace stays read-only for the fused pass. Each translation unit
// that holds fused kernels has its own array.
__device__ unsigned int kQueue[kQueueSlots];

__global__ void queue_reset_kernel(int slot) {
  if (threadIdx.x == 0) kQueue[slot] = 0u;
}

template <typename T, int D> struct Geom;
// bf16: K tile [64][D] and V^T tile [D][64], unpadded; 16-byte chunks are
// placed with an XOR swizzle so the MFMA operand reads hit distinct LDS banks.
// Two buffers: the next kept tile is loaded straight into LDS
// (buffer_load_dwordx4 ... lds) while the current one is computed.
template <int D> struct Geom<__bf16, D> {
  static constexpr int kKBytes = 64 * D * 2;
  static constexpr int kVBytes = D * 64 * 2;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kBuffers = 2;
};
template <int D> struct Geom<float, D> {
  static constexpr int kKPitch = D + 4;
  static constexpr int kVPitch = D + 4;
  static constexpr int kKBytes = 64 * kKPitch * 4;
  static constexpr int kVBytes = 64 * kVPitch * 4;
  static constexpr int kBufBytes = kKBytes + kVBytes;
  static constexpr int kBuffers = 1;
};

// LDS position (in 16-byte chunks) of chunk c of row r of a K tile: rows of
// D/8 chunks; the swizzle spreads the 16 rows one MFMA operand read touches
// over distinct banks.
template <int D> __device__ __forceinline__ int k_pos(int r, int c) {
  return r * (D / 8) + (c ^ (D == 128 ? (r & 15) : ((r >> 1) & 7)));
}
// LDS position of chunk kc (keys 8kc .. 8kc+7) of row d of a V^T tile.
__device__ __forceinline__ int v_pos(int d, int kc) { return d * 8 + (kc ^ ((d >> 1) & 7)); }


// LDS map. Static: two tile buffers A and B (separate objects, so the compiler
// can see that loads into one do not alias reads of the other); during
// routing they hold the G proxy rows (rows_per_buf rows each); the kept-set
// words are a third static object. Dynamic: [qa | acc | misc].
template <typename T, int D> struct Lds {
  static constexpr int kBuf = Geom<T, D>::kBufBytes;
  __host__ __device__ static int rows_per_buf(int nbp) { return kBuf / (4 * nbp); }
  __host__ __device__ static int qa(int, int) { return 0; }
  __host__ __device__ static int acc(int G, int nw) { return qa(G, nw) + 4 * D * kGMax; }
  __host__ __device__ static int misc(int G, int nw) { return acc(G, nw) + 4 * 4 * D * kGMax; }
  __host__ __device__ static int bytes(int G, int nw) { return misc(G, nw) + 4 * 64; }
};
// misc slots (floats)
constexpr int kRed = 0;          // [4 waves][8] reduction scratch
constexpr int kTot = 32;         // [8] reduction totals
constexpr int kTau = 40;         // [kGMax]
constexpr int kC2 = 44;          // [kGMax] correction max (base 2), -inf if none
constexpr int kL = 48;           // [kGMax] correction denominator 64 * sum w

constexpr float inv_sqrt(int d) { return d == 64 ? 0.125f : 0.08838834764831845f; }

// 2^x with the hardware v_exp_f32 (results below 2^-126 flush to 0, which a
// softmax weight can afford); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rows rescale their accumulators only when a new tile maximum exceeds the
// reference by more than this (base-2 exponent): weights then stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

// Sum over the workgroup of NV floats per thread; totals land in misc[kTot + v].
template <int NV>
__device__ inline void block_sum_n(float (&x)[NV], float* misc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = wave_sum(x[i]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) misc[kRed + w * 8 + i] = x[i];
  __syncthreads();
  if (threadIdx.x < NV)
    misc[kTot + threadIdx.x] = (misc[kRed + threadIdx.x] + misc[kRed + 8 + threadIdx.x]) +
                               (misc[kRed + 16 + threadIdx.x] + misc[kRed + 24 + threadIdx.x]);
  __syncthreads();
}
template <int NV>
__device__ inline void block_max_n(float (&x)[NV], float* misc) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = wave_max(x[i]);
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < NV; ++i) misc[kRed + w * 8 + i] = x[i];
  __syncthreads();
  if (threadIdx.x < NV)
    misc[kTot + threadIdx.x] = fmaxf(fmaxf(misc[kRed + threadIdx.x], misc[kRed + 8 + threadIdx.x]),
                                     fmaxf(misc[kRed + 16 + threadIdx.x], misc[kRed + 24 + threadIdx.x]));
  __syncthreads();
}

// Per-lane state of the exact phase (one query row, a quarter of its keys / dims).
template <typename T, int D> struct ExactState {
  static constexpr bool kBF = std::is_same<T, __bf16>::value;
  static constexpr int KS = D / 32;                 // k-steps of 32 head dims
  static constexpr int NACC = kBF ? D / 16 : 1;     // O^T tiles of 16 head dims
  static constexpr int NF = kBF ? 1 : D / 4;        // fp32 path: head dims per lane
  bf16x8 qop[kBF ? KS : 1];
  float qf[NF];
  f32x4 oacc[NACC];
  float of[NF];
  float mrow, lrow;
};

template <typename T, int D>
__device__ __forceinline__ void zero_state(ExactState<T, D>& st) {
  using S = ExactState<T, D>;
  st.mrow = -INFINITY;
  st.lrow = 0.f;
#pragma unroll
  for (int i = 0; i < S::NACC; ++i) st.oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < S::NF; ++i) st.of[i] = 0.f;
}

// this lane's part of its query row: MFMA operands (bf16) or D/4 floats (fp32)
template <typename T, int D>
__device__ __forceinline__ void load_q(ExactState<T, D>& st, const T* Qr, int lane) {
  using S = ExactState<T, D>;
  const int grp = lane >> 4;
  if constexpr (S::kBF) {
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) st.qop[ks] = *reinterpret_cast<const bf16x8*>(Qr + ks * 32 + grp * 8);
  } else {
#pragma unroll
    for (int e = 0; e < S::NF; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(Qr + grp * S::NF + e);
      st.qf[e] = x.x; st.qf[e + 1] = x.y; st.qf[e + 2] = x.z; st.qf[e + 3] = x.w;
    }
  }
}

typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef __attribute__((address_space(1))) const void gbl_ptr_t;

// Per-lane pieces of the tile loads. A tile region (K or V^T, 64 * D * 2
// bytes) is moved in slabs of 256 chunks of 16 bytes, one chunk per lane; the
// lane's source offset inside a slab is the same for every slab (the XOR
// swizzles depend on the row only through bits that do not change between
// slabs), slabs are 4096 bytes apart in both global memory and LDS, and the
// LDS destination of a wave is uniform (kept in a scalar register).
struct DmaLane {
  int k_off;         // byte offset of this lane's K chunk in slab 0 of a tile of the input K
  long long k_slab;  // bytes between slabs of the input K (16 or 32 rows; uniform)
  int kc_off;        // the same offset in a contiguous [64][D] tile (block summaries)
  int v_off;         // byte offset of this lane's V^T chunk in slab 0, or (low-memory
                     // mode) of its chunk of a row-major tile of the input V
  long long v_slab;  // bytes between slabs of that V source (uniform)
  int wave_lds;      // this wave's first LDS byte inside a slab (uniform)
};
// k_row, v_row: row strides of the input K and V in elements. VRM: V tiles
// row-major from the input V (same lane pattern and swizzle as K) instead of
// the pre-pass's V^T blocks.
template <int D, bool VRM>
__device__ __forceinline__ DmaLane dma_lane(int t, long long k_row, long long v_row) {
  DmaLane dl;
  constexpr int RPS = 4096 / (D * 2);   // rows per 4096-byte slab
  if constexpr (D == 128) {
    const int r = t >> 4, c = (t & 15) ^ (r & 15);          // rows of 16 chunks
    dl.k_off = (int)(r * k_row * 2) + c * 16;
    dl.kc_off = r * D * 2 + c * 16;
    if constexpr (VRM) dl.v_off = (int)(r * v_row * 2) + c * 16;
  } else {
    const int r = t >> 3, c = (t & 7) ^ ((r >> 1) & 7);     // rows of 8 chunks
    dl.k_off = (int)(r * k_row * 2) + c * 16;
    dl.kc_off = r * D * 2 + c * 16;
    if constexpr (VRM) dl.v_off = (int)(r * v_row * 2) + c * 16;
  }
  dl.k_slab = RPS * k_row * 2;
  if constexpr (VRM) {
    dl.v_slab = RPS * v_row * 2;
  } else {
    const int d = t >> 3, kc = (t & 7) ^ ((d >> 1) & 7);    // V^T rows of 8 chunks
    dl.v_off = d * 128 + kc * 16;
    dl.v_slab = 4096;
  }
  dl.wave_lds = __builtin_amdgcn_readfirstlane((t >> 6) * 1024);
  return dl;
}

// bf16: start loading the K tile and the V tile (transposed, or row-major in
// the low-memory mode) of key block j straight into LDS buffer `buf`. Each
// source is either the input tensor (row stride from the caller), a block of
// the V^T copy or a contiguous tile of block summaries: *_off is this lane's
// byte offset in the first slab of 4096 bytes of LDS and *_slab the byte
// distance between the slabs in the source. Completion is awaited with
// s_waitcnt vmcnt before the next barrier.
template <int D>
__device__ __forceinline__ void issue_tile(unsigned char* buf, const __bf16* Ksrc, int k_off, long long k_slab,
                                           const __bf16* Vsrc, int v_off, long long v_slab, const DmaLane& dl) {
  constexpr int NI = D / 32;   // slabs per region
  // Buffer-form loads: a scalar descriptor per region (base = the tile, size =
  // the tile's extent), this lane's fixed 32-bit offset and a scalar slab
  // offset, so the addresses need no per-lane arithmetic. The 4th descriptor
  // word selects 32-bit untyped data; accesses past the size read zeros.
  constexpr int kRsrcWord3 = 0x00020000;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Ksrc), (short)0, (int)(NI * k_slab), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(Vsrc), (short)0, (int)(NI * v_slab), kRsrcWord3);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t*)(buf + i * 4096 + dl.wave_lds), 16, (unsigned)k_off,
                                             (unsigned)(i * k_slab), 0, 0);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t*)(buf + Geom<__bf16, D>::kKBytes + i * 4096 + dl.wave_lds),
                                             16, (unsigned)v_off, (unsigned)(i * v_slab), 0, 0);
}

// fp32: stage the K and V tiles of key block j in LDS (synchronously)
template <int D>
__device__ __forceinline__ void commit_f32(float* stK, float* stV, const float* Kh, const float* Vh,
                                           long long k_row, long long v_row, int j, int t) {
  using Gm = Geom<float, D>;
  const float* Kj = Kh + (long long)j * kBlock * k_row;
  const float* Vj = Vh + (long long)j * kBlock * v_row;
  constexpr int CH = D / 4;
  for (int c = t; c < 64 * CH; c += 256) {
    const int r = c / CH, cc = c % CH;
    *reinterpret_cast<float4*>(stK + r * Gm::kKPitch + cc * 4) =
        reinterpret_cast<const float4*>(Kj + (long long)r * k_row)[cc];
    *reinterpret_cast<float4*>(stV + r * Gm::kVPitch + cc * 4) =
        reinterpret_cast<const float4*>(Vj + (long long)r * v_row)[cc];
  }
}

// Byte offsets of this lane's MFMA operand reads inside a tile buffer. The
// swizzles depend on the row only through lane % 16 (every 16-row sub-tile
// starts at a multiple of 16), so one offset per k-step serves all
// sub-tiles, which differ by compile-time displacements.
//
// VRM (low-memory mode): V tiles are row-major in LDS, with the K tiles'
// swizzle, and each P.V A operand is gathered by two transposing reads
// (ds_read_b64_tr_b16): within each group of 16 lanes, result lane i, element
// e is element i % 4 of the 8 bytes source lane 4e + i / 4 points at. For
// d-tile dt (16 head dims) and keys 32ks + 16h + 4g + e (g = lane / 16, the key
// order of P), source lane 16g + j points at row 32ks + 16h + 4g + j / 4, head
// dims 16dt + 4(j % 4) .. +3; in a swizzled row that is the address of d-tile
// 0 with byte bits 5-7 flipped by dt, and rows 16 apart keep the swizzle.
template <int D, bool VRM = false> struct LaneOfs {
  static constexpr int kNV = VRM ? D / 16 : 2;
  int k[D / 32];   // K operand, k-step ks: row lane%16 of sub-tile 0, chunk 4ks + lane/16
  int v[kNV];      // V^T operand, k-step ks: row lane%16 of d-tile 0, chunk 4ks + lane/16;
                   // VRM: d-tile dt, the transposing read of k-step 0, half 0
  __device__ __forceinline__ explicit LaneOfs(int lane) {
    const int l16 = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) k[ks] = 16 * k_pos<D>(l16, ks * 4 + grp);
    if constexpr (VRM) {
      const int r0 = 4 * grp + (l16 >> 2);   // row within the 16-key half
#pragma unroll
      for (int dt = 0; dt < kNV; ++dt)
        v[dt] = Geom<__bf16, D>::kKBytes + 16 * k_pos<D>(r0, 2 * dt + ((lane >> 1) & 1)) + 8 * (lane & 1);
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) v[ks] = Geom<__bf16, D>::kKBytes + 16 * v_pos(l16, ks * 4 + grp);
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// transposing LDS read of four bf16 at byte offset `off` of `buf` (see LaneOfs)
__device__ __forceinline__ s16x4 tr_read(const unsigned char* buf, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) unsigned char*)(const_cast<unsigned char*>(buf)) + off));
}

// One tile of 64 keys for one query block of this wave: S^T = K Q^T, online
// softmax in base 2, O^T += V^T P^T.
// VIRT: a tile of block summaries (per-row correction): the 64 "keys" are the
// block means k_bar_j of 64 key blocks, each standing for 64 equal tokens
// (base-2 logit + log2(64) = 6), values v_bar_j; key blocks whose bit is set
// in `excl` (kept exactly, or past n_b) get weight zero.
// XO: operand offsets of k-steps ks > 0 formed in the tile from those of
// k-step 0 (4 fewer registers held across the walk, 4 more VALU per tile):
// used where the register budget is tightest (the per-row correction).
template <int D, bool VIRT = false, bool XO = false, bool VRM = false>
__device__ __forceinline__ void tile_bf16(ExactState<__bf16, D>& st, const unsigned char* buf,
                                          const LaneOfs<D, VRM>& lo, uint64_t excl = 0) {
  using S = ExactState<__bf16, D>;
  constexpr int NV = LaneOfs<D, VRM>::kNV;
  // The XOR swizzles make the chunk index of k-step ks that of k-step 0 with
  // bits 2-3 flipped by ks, i.e. byte offset bits 6-7 (K) or bit 6 (V^T), and
  // (VRM) the V offset of d-tile dt that of d-tile 0 with bits 5-7 flipped by
  // dt; the empty asm keeps the compiler from hoisting the derived offsets
  // out of the walk.
  int ko[S::KS], vo[NV];
  if constexpr (XO) {
    int k0 = lo.k[0], v0 = lo.v[0];
    asm volatile("" : "+v"(k0), "+v"(v0));
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) ko[ks] = k0 ^ (64 * ks);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      vo[i] = VRM ? (v0 ^ (32 * i)) : Geom<__bf16, D>::kKBytes + ((v0 - Geom<__bf16, D>::kKBytes) ^ (64 * i));
  } else {
#pragma unroll
    for (int ks = 0; ks < S::KS; ++ks) ko[ks] = lo.k[ks];
#pragma unroll
    for (int i = 0; i < NV; ++i) vo[i] = lo.v[i];
  }
  constexpr float kScale2 = inv_sqrt(D) * kLog2e;   // logit -> base-2 exponent
  constexpr float kOff = VIRT ? 6.0f : 0.0f;        // log2 of the multiplicity
  // S^T (64 keys x 16 queries): 4 key sub-tiles of 16 rows of D/8 chunks
  // (16*D*2 bytes apart). K-step outer, sub-tile inner: four independent
  // accumulation chains, and the operands of k-step ks+1 are read while the
  // MFMAs of k-step ks run.
  f32x4 s[4];
  bf16x8 ka[2][4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    ka[0][kt] = *reinterpret_cast<const bf16x8*>(buf + ko[0] + kt * 16 * D * 2);
  }
#pragma unroll
  for (int ks = 0; ks < S::KS; ++ks) {
    if (ks + 1 < S::KS) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        ka[(ks + 1) & 1][kt] = *reinterpret_cast<const bf16x8*>(buf + ko[ks + 1] + kt * 16 * D * 2);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
      s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[ks & 1][kt], st.qop[ks], s[kt], 0, 0, 0);
  }
  if constexpr (VIRT) {
    // the lane's 16 keys are 16kt + 4*(lane/16) + i: gather their exclusion
    // bits into one 16-bit lane mask (excl is uniform, in scalar registers)
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)excl);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(excl >> 32));
    const int sh = 4 * ((threadIdx.x & 63) >> 4);
    const uint32_t m16 = ((lo >> sh) & 0xFu) | (((lo >> (16 + sh)) & 0xFu) << 4) |
                         (((hi >> sh) & 0xFu) << 8) | (((hi >> (16 + sh)) & 0xFu) << 12);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if ((m16 >> (4 * kt + i)) & 1u) s[kt][i] = -INFINITY;
  }
  // Online softmax: the lane holds keys 16kt + (lane/16)*4 + i of its query
  // row. A row's reference moves only when the tile maximum exceeds it by the
  // slack. Each lane first tests its own 16 values; only when some lane of
  // the wave passes are the four lanes of each row reconciled (row maximum
  // over the tile, the same on the row's four lanes, so they stay in step).
  float lmax = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) lmax = fmaxf(lmax, s[kt][i]);
  lmax = lmax * kScale2 + kOff;
  if (__ballot(lmax > st.mrow + kRescaleSlack)) {
    const float tmax = quad16_max(lmax);
    const bool grow = tmax > st.mrow + kRescaleSlack;
    const float mnew = grow ? tmax : st.mrow;
    const float alpha = fast_exp2(st.mrow - mnew);   // 0 on the first tile, 1 if !grow
    st.lrow *= alpha;
#pragma unroll
    for (int dt = 0; dt < S::NACC; ++dt) st.oacc[dt] *= alpha;
    st.mrow = mnew;
  }
  const float mref = st.mrow;
  bf16x8 pop[2];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pop[kt >> 1][(kt & 1) * 4 + i] = to_bf16(fast_exp2(__builtin_fmaf(s[kt][i], kScale2, kOff - mref)));
  // the row sum adds the bf16 weights that enter the P V product, two per
  // dot2 instruction (products by 1 are exact, accumulation in fp32)
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float l = st.lrow;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      l = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pop[ks][e], pop[ks][e + 1]}, ones, l, false);
  st.lrow = l;
  // O^T (d x 16 queries) += V^T (d x 64 keys) P^T in two k-steps of 32 keys;
  // V^T columns are stored in operand order; d-tiles are 16 rows of 8 chunks
  // = 2048 bytes apart. VRM: each A operand is two transposing reads of the
  // row-major V tile (keys 32ks + 4g + 0..3, then the same + 16; rows 16
  // apart are 32 D bytes apart).
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int dt = 0; dt < S::NACC; ++dt) {
      bf16x8 a;
      if constexpr (VRM) {
        constexpr int kRow = 2 * D;
        const s16x4 lo4 = tr_read(buf, vo[dt] + 32 * ks * kRow);
        const s16x4 hi4 = tr_read(buf, vo[dt] + (32 * ks + 16) * kRow);
        a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      } else {
        a = *reinterpret_cast<const bf16x8*>(buf + vo[ks] + dt * 2048);
      }
      st.oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pop[ks], st.oacc[dt], 0, 0, 0);
    }
  }
}

// One tile of 64 keys for one query block, fp32: 4 lanes per query row, each
// a quarter of the head dims; dot products and the weighted sum of V on the
// VALU from LDS-staged K and V; online softmax in base 2.
template <int D, bool VIRT = false>
__device__ __forceinline__ void tile_f32(ExactState<float, D>& st, const unsigned char* buf, int lane,
                                         uint64_t excl = 0) {
  using S = ExactState<float, D>;
  using Gm = Geom<float, D>;
  constexpr float kScale2 = inv_sqrt(D) * kLog2e;   // logit -> base-2 exponent
  constexpr float kOff = VIRT ? 6.0f : 0.0f;        // log2 of the multiplicity (block summaries)
  const int grp = lane >> 4;
  {
    const float* stK = reinterpret_cast<const float*>(buf);
    const float* stV = reinterpret_cast<const float*>(buf + Gm::kKBytes);
    float sv[64];
    float tmax = -INFINITY;
#pragma unroll
    for (int key = 0; key < 64; ++key) {
      const float* kr = stK + key * Gm::kKPitch + grp * S::NF;
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < S::NF; ++e) a += st.qf[e] * kr[e];
      a += __shfl_xor(a, 16, 64);
      a += __shfl_xor(a, 32, 64);
      sv[key] = (VIRT && ((excl >> key) & 1ull)) ? -INFINITY : a * kScale2 + kOff;
      tmax = fmaxf(tmax, sv[key]);
    }
    const float mnew = fmaxf(st.mrow, tmax);
    const float alpha = fast_exp2(st.mrow - mnew);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < S::NF; ++e) st.of[e] *= alpha;
#pragma unroll
    for (int key = 0; key < 64; ++key) {
      const float pvv = fast_exp2(sv[key] - mnew);
      psum += pvv;
      const float* vr = stV + key * Gm::kVPitch + grp * S::NF;
#pragma unroll
      for (int e = 0; e < S::NF; ++e) st.of[e] += pvv * vr[e];
    }
    st.lrow = st.lrow * alpha + psum;
    st.mrow = mnew;
  }
}

// out = (O 2^(m-M) + A 2^(c-M)) / (l 2^(m-M) + L 2^(c-M)) for query block qb
template <typename T, int D>
__device__ __forceinline__ void epilogue(ExactState<T, D>& st, const FusedParams& p, long long bh, int qb,
                                         int g, int row, int lane, const float* qa, const float* misc) {
  using S = ExactState<T, D>;
  const int grp = lane >> 4;
  float l = st.lrow;
  if constexpr (S::kBF) l = quad16_sum(l);   // lanes of one row held partial key sums
  const float c2 = misc[kC2 + g], Lg = misc[kL + g];
  const float M = fmaxf(st.mrow, c2);
  const float fo = (st.mrow == -INFINITY) ? 0.f : fast_exp2(st.mrow - M);
  const float fc = (c2 == -INFINITY) ? 0.f : fast_exp2(c2 - M);
  const float den = l * fo + Lg * fc;
  const float inv = den > 0.f ? 1.0f / den : 0.f;
  T* orow = static_cast<T*>(p.out) + (bh / p.H) * p.os.b + (bh % p.H) * p.os.h +
            ((long long)qb * kBlock + row) * p.os.n;
  if constexpr (S::kBF) {
#pragma unroll
    for (int dt = 0; dt < S::NACC; ++dt) {
      const int d0 = dt * 16 + grp * 4;
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (c2 > -INFINITY) ? qa[(d0 + i) * kGMax + g] * fc : 0.f;
        o[i] = (st.oacc[dt][i] * fo + a) * inv;
      }
      bf16x4 ob = {to_bf16(o[0]), to_bf16(o[1]), to_bf16(o[2]), to_bf16(o[3])};
      *reinterpret_cast<bf16x4*>(orow + d0) = ob;
    }
  } else {
#pragma unroll
    for (int e = 0; e < S::NF; e += 4) {
      const int d0 = grp * S::NF + e;
      float4 o;
      float* op = &o.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = (c2 > -INFINITY) ? qa[(d0 + i) * kGMax + g] * fc : 0.f;
        op[i] = (st.of[e + i] * fo + a) * inv;
      }
      *reinterpret_cast<float4*>(orow + d0) = o;
    }
  }
}

// Kernel modes: routing without / with the correction (block-level logit), a
// caller-given block mask (plain block-sparse attention: no routing, no
// correction), or routing with the per-row correction logit (the unselected
// blocks enter as tiles of block summaries in the walk).
constexpr int kModeRoute = 0, kModeCorr = 1, kModeGiven = 2, kModeCorrRow = 3;

// LM (bf16 only): low-memory mode, value tiles from the input V (row-major,
// transposing operand reads) instead of the pre-pass's V^T copy.
template <typename T, int D, int MODE, bool LM = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_kernel(FusedParams p) {
  constexpr bool CORR = MODE == kModeCorr;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  using Gm = Geom<T, D>;
  using L = Lds<T, D>;
  constexpr float kInvSqrtD = inv_sqrt(D);

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n_b = p.n_b, nbp = p.n_b_pad, n_words = p.n_words;

  // Work items (G consecutive query blocks of one head). The first
  // BH - dyn_heads heads are mapped statically and XCD-aware: the hardware
  // deals workgroups round-robin over the 8 XCDs; each head's n_groups items
  // are cut into 8 contiguous runs, run x going to XCD x, and heads are taken
  // in order, so all XCDs work on the same head at a time (its K and V^T stay
  // in the shared Infinity Cache) and each XCD's L2 sees neighbouring query
  // blocks, which keep similar key blocks. The items of the last dyn_heads
  // heads form a queue served by the remaining workgroups (workers, twice as
  // many as those items): each takes at most one item from a device counter,
  // so an XCD that finishes its static share early starts its workers early
  // and takes more of the end of the launch; workers that find the queue
  // empty leave at once.
  __shared__ int item_slot;
  const long long wgid = blockIdx.x;
  long long bh;
  int grp_id;
  if (wgid < p.n_static_wg) {
    const long long r = wgid >> 3;
    bh = r / p.per_xcd;
    grp_id = (int)((wgid & 7) * p.per_xcd + (r - bh * p.per_xcd));
    if (bh >= p.BH - p.dyn_heads || grp_id >= p.n_groups) return;   // uniform over the workgroup
  } else {
    if (t == 0) item_slot = (int)atomicAdd(&kQueue[p.qslot], 1u);
    __syncthreads();
    const int slot = __builtin_amdgcn_readfirstlane(item_slot);
    if (slot >= p.dyn_heads * p.n_groups) return;   // queue empty: uniform over the workgroup
    bh = p.BH - p.dyn_heads + slot / p.n_groups;
    grp_id = slot % p.n_groups;
  }
  const int qi0 = grp_id * p.G;
  const int nG = min(p.G, n_b - qi0);
  // optional work-item timing (debug): 100 MHz constant clock at start and end
  const unsigned long long clk0 = p.item_clock ? __builtin_amdgcn_s_memrealtime() : 0ull;

  constexpr bool kBF = std::is_same<T, __bf16>::value;
  __shared__ __attribute__((aligned(16))) unsigned char sbufA[Gm::kBufBytes];
  __shared__ __attribute__((aligned(16))) unsigned char sbufB[Gm::kBuffers == 2 ? Gm::kBufBytes : 16];
  // kept-set words [G][n_words]: a static object of its own, so the compiler
  // sees that the LDS-DMA loads in flight do not write them
  __shared__ uint64_t masks[kGMax * (kMaxBlocks / 64)];
  float* qa = reinterpret_cast<float*>(lds + L::qa(p.G, n_words));          // [D][kGMax]
  float* acc = reinterpret_cast<float*>(lds + L::acc(p.G, n_words));        // [4][kGMax][D]
  float* misc = reinterpret_cast<float*>(lds + L::misc(p.G, n_words));
  // proxy rows of the routing phase, overlaid on the tile buffers
  float* shr[kGMax];
  {
    const int rpb = L::rows_per_buf(nbp);
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
      shr[g] = g < rpb ? reinterpret_cast<float*>(sbufA) + g * nbp
                       : reinterpret_cast<float*>(sbufB) + (g - rpb) * nbp;
  }

  const long long ib = bh / p.H, ih = bh % p.H;
  const T* Qh = static_cast<const T*>(p.q) + ib * p.qs.b + ih * p.qs.h;   // row t at Qh + t * qs.n
  const T* Kh = static_cast<const T*>(p.k) + ib * p.ks.b + ih * p.ks.h;
  const T* Vh = static_cast<const T*>(p.v) + ib * p.vs.b + ih * p.vs.h;

  if constexpr (MODE == kModeGiven) {
    // ---- caller-given selection: the G blocks' mask words into LDS ----------
    for (int e = t; e < nG * n_words; e += 256) {
      const int g = e / n_words, wi = e % n_words;
      uint64_t word = p.mask_in[(bh * n_b + qi0 + g) * (long long)n_words + wi];
      if (wi == n_words - 1 && (n_b & 63)) word &= (1ull << (n_b & 63)) - 1;   // bits past n_b ignored
      masks[g * n_words + wi] = word;
    }
    if (t < kGMax) {
      misc[kC2 + t] = -INFINITY;   // no correction term
      misc[kL + t] = 0.f;
    }
    __syncthreads();
    if (p.kept_per_row && t < nG) {
      int c = 0;
      for (int wi = 0; wi < n_words; ++wi) c += __popcll(masks[t * n_words + wi]);
      p.kept_per_row[bh * n_b + qi0 + t] = c;
    }
  } else {
  // ---- 1. q_bar of the G query blocks ---------------------------------------
  {
    using V16 = Vec16<T>;
    constexpr int E = V16::kN, CH = D / E, RPT = 64 * CH / 256, RSTEP = 256 / CH;
    const int cc = t % CH, r0 = t / CH;
    // every block's loads first (one round of L2/HBM latency for the group)
    typename V16::raw rq[kGMax][RPT];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      if (g < nG) {
        const T* Qb = Qh + (long long)(qi0 + g) * kBlock * p.qs.n;
#pragma unroll
        for (int i = 0; i < RPT; ++i)
          rq[g][i] = reinterpret_cast<const typename V16::raw*>(Qb + (long long)(r0 + RSTEP * i) * p.qs.n)[cc];
      }
    }
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      if (g < nG) {
        float s[E];
#pragma unroll
        for (int e = 0; e < E; ++e) s[e] = 0.f;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          float f[E];
          V16::to_float(rq[g][i], f);
#pragma unroll
          for (int e = 0; e < E; ++e) s[e] += f[e];
        }
#pragma unroll
        for (int o = CH; o < 64; o <<= 1)
#pragma unroll
          for (int e = 0; e < E; ++e) s[e] += __shfl_xor(s[e], o, 64);
        if (lane < CH)
#pragma unroll
          for (int e = 0; e < E; ++e) acc[(w * kGMax + g) * D + cc * E + e] = s[e];
      }
    }
  }
  __syncthreads();
  if (t < D) {
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      float s = 0.f;
      if (g < nG)
        s = ((acc[(0 * kGMax + g) * D + t] + acc[(1 * kGMax + g) * D + t]) +
             (acc[(2 * kGMax + g) * D + t] + acc[(3 * kGMax + g) * D + t])) * (1.0f / kBlock);
      qa[t * kGMax + g] = s;   // zero for g >= nG: those proxy rows are never used
    }
  }
  __syncthreads();

  // ---- 2. tau = mu + beta sigma for each block (closed form) ----------------
  {
    const float* C = p.kcov + (size_t)bh * D * D;
    const float* m = p.kmean + (size_t)bh * D;
    // thread (part, r4): rows r4 .. r4+3 of C q_bar over CP consecutive c,
    // one float4 of C per c, all CP loads in flight at once
    constexpr int RQ = D / 4, NP = 256 / RQ, CP = D / NP;
    const int r4 = 4 * (t % RQ), part = t / RQ;
    float4 cv[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) cv[i] = *reinterpret_cast<const float4*>(C + (size_t)(part * CP + i) * D + r4);
    float y[kGMax][4];
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) y[g][e] = 0.f;
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      const float4 qv = *reinterpret_cast<const float4*>(qa + (part * CP + i) * kGMax);
      const float qg[4] = {qv.x, qv.y, qv.z, qv.w};
      const float cr[4] = {cv[i].x, cv[i].y, cv[i].z, cv[i].w};
#pragma unroll
      for (int g = 0; g < kGMax; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) y[g][e] += cr[e] * qg[g];
    }
    const float4 mv = part == 0 ? *reinterpret_cast<const float4*>(m + r4) : make_float4(0.f, 0.f, 0.f, 0.f);
    const float mr[4] = {mv.x, mv.y, mv.z, mv.w};
    float v8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 qr = *reinterpret_cast<const float4*>(qa + (r4 + e) * kGMax);
      const float qe[4] = {qr.x, qr.y, qr.z, qr.w};
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        v8[g] += qe[g] * y[g][e];
        v8[4 + g] += qe[g] * mr[e];
      }
    }
    block_sum_n<8>(v8, misc);
    if (t < nG) {
      const float qcq = misc[kTot + t], qm = misc[kTot + 4 + t];
      const float mu = qm * kInvSqrtD;
      const float sigma = sqrtf(fmaxf(qcq, 0.f) * (1.0f / D));
      float tau;
      if (p.beta_mode == kBetaMinusInf) tau = -INFINITY;
      else if (p.beta_mode == kBetaPlusInf) tau = INFINITY;
      else tau = mu + p.beta * sigma;
      misc[kTau + t] = tau;
    }
  }

  // ---- 3a. outer loop: proxy scores of every key block for the G blocks ------
  {
    const float* kt = p.kbar_t + (size_t)bh * D * nbp;
    for (int j4 = 4 * t; j4 < n_b; j4 += 1024) {
      float a[kGMax][4];
#pragma unroll
      for (int g = 0; g < kGMax; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[g][e] = 0.f;
#pragma unroll 16
      for (int c = 0; c < D; ++c) {
        const float4 kv = *reinterpret_cast<const float4*>(kt + (size_t)c * nbp + j4);
        const float4 qv = *reinterpret_cast<const float4*>(qa + c * kGMax);
        const float qg[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int g = 0; g < kGMax; ++g) {
          a[g][0] += qg[g] * kv.x; a[g][1] += qg[g] * kv.y;
          a[g][2] += qg[g] * kv.z; a[g][3] += qg[g] * kv.w;
        }
      }
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        if (g < nG) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (j4 + e < n_b) shr[g][j4 + e] = a[g][e] * kInvSqrtD;
        }
      }
    }
  }
  __syncthreads();

  // ---- 3b. strict test against tau -> one 64-bit word per 64 key blocks ------
  {
    const int t0 = n_b - p.text_blocks;
    float cmax[kGMax] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    float kept[kGMax] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      if (g < nG) {
        const float tau = misc[kTau + g];
        for (int wi = w; wi < n_words; wi += 4) {
          const int j = wi * 64 + lane;
          const bool valid = j < n_b;
          const float s = valid ? shr[g][j] : 0.f;
          // text key blocks and text query blocks (joint attention) are always exact
          const bool keep = valid && (s > tau || j >= t0 || qi0 + g >= t0);
          const uint64_t word = __ballot(keep);
          if (valid && !keep) cmax[g] = fmaxf(cmax[g], s);
          if (lane == 0) masks[g * n_words + wi] = word;
          kept[g] += (lane == 0) ? (float)__popcll(word) : 0.f;
        }
      }
    }
    block_max_n<kGMax>(cmax, misc);
    if (t < kGMax) {
      misc[kC2 + t] = (CORR && misc[kTot + t] > -INFINITY) ? misc[kTot + t] * kLog2e : -INFINITY;
      misc[kL + t] = 0.f;
    }
    block_sum_n<kGMax>(kept, misc);
    for (int g = 0; g < nG; ++g) {
      const long long qrow = bh * n_b + qi0 + g;
      if (t == 0) {
        if (p.kept_per_row) p.kept_per_row[qrow] = (int)misc[kTot + g];
        if (p.tau_out) p.tau_out[qrow] = misc[kTau + g];
      }
      if (p.mask_bits)
        for (int wi = t; wi < n_words; wi += 256) p.mask_bits[qrow * n_words + wi] = masks[g * n_words + wi];
    }
  }

  // ---- 4. correction: unselected blocks as 64 virtual tokens ----------------
  if constexpr (CORR && kBF) {
    // bf16 inputs: the weights w_gj = 2^(s_hat_gj log2e - c_g) of the
    // unselected blocks are rounded to bf16 (the row sum L adds the same
    // rounded weights), and A_g = 64 sum_j w_gj v_bar_j runs on MFMA against
    // the bf16 tiles of v_bar^T that the pre-pass writes for the per-row
    // correction (columns of key blocks in the P-operand order of the walk).
    float c2[kGMax];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) c2[g] = misc[kC2 + g];
    const int nw64 = n_words * 64;
    float wr[kGMax][kMaxBlocks / 256];
    float lp[kGMax] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kMaxBlocks / 256; ++i) {
      const int j = t + 256 * i;
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        float wj = 0.f;
        if (j < n_b && g < nG) {
          const bool keep = (masks[g * n_words + (j >> 6)] >> (j & 63)) & 1ull;
          if (!keep && c2[g] != -INFINITY)
            wj = (float)to_bf16(fast_exp2(shr[g][j] * kLog2e - c2[g]));
        }
        wr[g][i] = wj;
        lp[g] += wj;
      }
    }
    block_sum_n<kGMax>(lp, misc);   // barriers: every proxy row has been read
    if (t < kGMax) misc[kL + t] = misc[kTot + t] * (float)kBlock;
    // bf16 weights in the tile column order: key block 64c + r sits at column
    // 64c + q(r), q the inverse of the column -> key map of v_bar^T tiles;
    // rows 0, 1 in the first tile buffer, rows 2, 3 in the second (zero past n_b)
    auto wrow = [&](int g) -> __bf16* {
      return reinterpret_cast<__bf16*>(g < 2 ? sbufA : sbufB) + (g & 1) * nw64;
    };
#pragma unroll
    for (int i = 0; i < kMaxBlocks / 256; ++i) {
      const int j = t + 256 * i;
      if (j < nw64) {
        const int r = j & 63, h = r >> 5, r32 = r & 31;
        const int q = r32 < 16 ? 32 * h + 8 * (r32 >> 2) + (r32 & 3)
                               : 32 * h + 8 * ((r32 - 16) >> 2) + 4 + (r32 & 3);
#pragma unroll
        for (int g = 0; g < kGMax; ++g) wrow(g)[(j & ~63) + q] = to_bf16(wr[g][i]);
      }
    }
    __syncthreads();
    // A^T (d x 16 columns, column g < nG) += v_bar^T (d x 32 key blocks) W^T,
    // k-steps of 32 key blocks dealt round-robin to the 4 waves
    {
      const int l16 = lane & 15, grp = lane >> 4;
      const __bf16* vbt = p.vbar_t + (size_t)bh * n_words * D * 64;
      f32x4 o[D / 16];
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const bf16x8 zero8 = {};
      // k-steps of 32 key blocks, four per wave at a time: the L2 loads of
      // their v_bar^T operands are all issued before the first MFMA
      const int nks = 2 * n_words;
      int ks = w;
      for (; ks + 12 < nks; ks += 16) {
        bf16x8 av[4][D / 16], bw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k1 = ks + 4 * u;
          const __bf16* vrow = vbt + ((size_t)(k1 >> 1) * D + l16) * 64 + 32 * (k1 & 1) + 8 * grp;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            av[u][dt] = *reinterpret_cast<const bf16x8*>(vrow + (size_t)dt * 16 * 64);
          bw[u] = l16 < nG ? *reinterpret_cast<const bf16x8*>(wrow(l16 < 4 ? l16 : 0) + 32 * k1 + 8 * grp)
                           : zero8;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][dt], bw[u], o[dt], 0, 0, 0);
      }
      for (; ks < nks; ks += 4) {
        const bf16x8 bw = l16 < nG ? *reinterpret_cast<const bf16x8*>(wrow(l16 < 4 ? l16 : 0) + 32 * ks + 8 * grp)
                                   : zero8;
        const __bf16* vrow = vbt + ((size_t)(ks >> 1) * D + l16) * 64 + 32 * (ks & 1) + 8 * grp;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(vrow + (size_t)dt * 16 * 64);
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bw, o[dt], 0, 0, 0);
        }
      }
      // lane holds A^T[16dt + 4 grp + i][g = l16]
      if (l16 < nG) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[(w * kGMax + l16) * D + 16 * dt + 4 * grp + i] = o[dt][i] * (float)kBlock;
      }
    }
    __syncthreads();
    if (t < D) {
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        const float s = (acc[(0 * kGMax + g) * D + t] + acc[(1 * kGMax + g) * D + t]) +
                        (acc[(2 * kGMax + g) * D + t] + acc[(3 * kGMax + g) * D + t]);
        qa[t * kGMax + g] = s;   // q_bar is no longer needed: qa now holds A
      }
    }
  } else if constexpr (CORR) {
    float c2[kGMax];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) c2[g] = misc[kC2 + g];
    float lp[kGMax] = {0.f, 0.f, 0.f, 0.f};
    for (int j = t; j < n_b; j += 256) {
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        if (g < nG) {
          const bool keep = (masks[g * n_words + (j >> 6)] >> (j & 63)) & 1ull;
          const float wj = (keep || c2[g] == -INFINITY) ? 0.f : fast_exp2(shr[g][j] * kLog2e - c2[g]);
          shr[g][j] = wj;
          lp[g] += wj;
        }
      }
    }
    block_sum_n<kGMax>(lp, misc);   // barrier: the weights are complete
    if (t < kGMax) misc[kL + t] = misc[kTot + t] * (float)kBlock;
    // A_g = sum_j w_gj vsum_j: lane (jr, c4) takes columns 4*c4 .. 4*c4+3 of
    // key blocks j = jr, jr + RG, ...; each float4 of vsum serves all G blocks
    constexpr int C4 = D / 4, RG = 256 / C4;
    const int c4 = t % C4, jr = t / C4;
    const float4* vs = reinterpret_cast<const float4*>(p.vsum + (size_t)bh * n_b * D) + c4;
    f32x4 a[kGMax];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) a[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    // unconditional loads (kept blocks carry weight 0), so the unrolled
    // iterations keep several L2 loads in flight
#pragma unroll 8
    for (int j = jr; j < n_b; j += RG) {
      const float4 x = vs[(size_t)j * C4];
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        const float wj = g < nG ? shr[g][j] : 0.f;
        a[g][0] += wj * x.x; a[g][1] += wj * x.y;
        a[g][2] += wj * x.z; a[g][3] += wj * x.w;
      }
    }
    // fold the row groups of a wave (lanes c4 + C4*r), then the 4 waves via LDS
#pragma unroll
    for (int o = C4; o < 64; o <<= 1)
#pragma unroll
      for (int g = 0; g < kGMax; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) a[g][e] += __shfl_xor(a[g][e], o, 64);
    if (lane < C4)
#pragma unroll
      for (int g = 0; g < kGMax; ++g)
        *reinterpret_cast<f32x4*>(acc + (w * kGMax + g) * D + 4 * c4) = a[g];
    __syncthreads();
    if (t < D) {
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        const float s = (acc[(0 * kGMax + g) * D + t] + acc[(1 * kGMax + g) * D + t]) +
                        (acc[(2 * kGMax + g) * D + t] + acc[(3 * kGMax + g) * D + t]);
        qa[t * kGMax + g] = s;   // q_bar is no longer needed: qa now holds A
      }
    }
  }
  }   // routing
  __syncthreads();   // masks, A, L, c2 visible; the proxy rows are dead

  // ---- 5. inner loop: exact attention on the kept tiles ---------------------
  const int row = 16 * w + (lane & 15);   // this lane's query row within a block
  if constexpr (kBF) {
    // The G blocks' kept lists are walked together in ascending key-block
    // order: each tile of their union is loaded once and computed for every
    // block that keeps it; the G online-softmax states stay in registers.
    // One barrier per union tile: wait for this lane's loads of tile j,
    // barrier (all lanes' loads landed; every wave finished the previous tile,
    // so the other buffer is free), start loading the next union tile into
    // it, compute tile j.
    const LaneOfs<D, LM> lofs(lane);
    const DmaLane dl = dma_lane<D, LM>(t, p.ks.n, p.vs.n);
    constexpr bool kXO = MODE == kModeCorrRow;   // register budget: see tile_bf16
    ExactState<T, D> sts[kGMax];
#pragma unroll
    for (int g = 0; g < kGMax; ++g) {
      zero_state<T, D>(sts[g]);
      if (g < nG) load_q<T, D>(sts[g], Qh + ((long long)(qi0 + g) * kBlock + row) * p.qs.n, lane);
    }
    // The walk keeps the G blocks' mask words of one 64-block word index (cw)
    // and their union in scalar registers; LDS is read again only when the
    // walk moves on to the next word.
    uint64_t wm[kGMax];
    uint64_t uw = 0;
    int cw = -1;
    auto load_word = [&](int wi) {
      uw = 0;
#pragma unroll
      for (int g = 0; g < kGMax; ++g) {
        const uint64_t x = g < nG ? masks[g * n_words + wi] : 0ull;
        wm[g] = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(x >> 32)) << 32) |
                (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)x);
        uw |= wm[g];
      }
      cw = wi;
    };
    auto union_next = [&](int j) -> int {   // next key block after j kept by any block
      int wi = (j + 1) >> 6;
      if (wi >= n_words) return -1;
      if (wi != cw) load_word(wi);
      uint64_t word = uw & (~0ull << ((j + 1) & 63));
      while (!word) {
        if (++wi >= n_words) return -1;
        load_word(wi);
        word = uw;
      }
      return wi * 64 + (int)__builtin_ctzll(word);
    };
    // value tile of key block j: a block of the V^T copy, or (LM) rows of V
    auto vtile = [&](int jj) -> const __bf16* {
      if constexpr (LM) return reinterpret_cast<const __bf16*>(Vh) + (long long)jj * kBlock * p.vs.n;
      else return p.vt + ((size_t)bh * n_b + jj) * D * 64;
    };
// s_waitcnt vmcnt(0) through the builtin, so the compiler's own wait tracking
// knows the tile loads have landed (gfx9 encoding: vmcnt in bits 3:0, expcnt
// 6:4 and lgkmcnt 11:8 left at their maxima)
#define SOL_WAIT_VM() __builtin_amdgcn_s_waitcnt(0xF70)
#define SOL_STEP(CURB, NEXTB)                                                     \
    {                                                                             \
      /* j lies in word cw (union_next found it there) */                       \
      unsigned keep = 0;                                                          \
      _Pragma("unroll") for (int g = 0; g < kGMax; ++g)                           \
        keep |= (unsigned)((wm[g] >> (j & 63)) & 1ull) << g;                      \
      const int nj = union_next(j);                                               \
      /* this lane's loads of tile j have landed; the tile loop writes LDS  */    \
      /* only through those loads and every read of the other buffer was    */    \
      /* consumed by an MFMA, so a bare barrier suffices                    */    \
      SOL_WAIT_VM();                                                              \
      asm volatile("" ::: "memory");                                              \
      __builtin_amdgcn_s_barrier();                                               \
      asm volatile("" ::: "memory");                                              \
      if (nj >= 0)                                                                \
        issue_tile<D>(NEXTB, Kh + (long long)nj * kBlock * p.ks.n, dl.k_off, dl.k_slab, vtile(nj), dl.v_off, dl.v_slab, dl); \
      _Pragma("unroll") for (int g = 0; g < kGMax; ++g)                           \
        if (keep & (1u << g)) tile_bf16<D, false, kXO, LM>(sts[g], CURB, lofs);  \
      j = nj;                                                                     \
    }
    int j = union_next(-1);
    if (j >= 0) issue_tile<D>(sbufA, Kh + (long long)j * kBlock * p.ks.n, dl.k_off, dl.k_slab, vtile(j), dl.v_off, dl.v_slab, dl);
    while (j >= 0) {
      SOL_STEP(sbufA, sbufB)
      if (j < 0) break;
      SOL_STEP(sbufB, sbufA)
    }
    if constexpr (MODE == kModeCorrRow) {
      // Per-row correction: the n_words tiles of block summaries (k_bar_j and
      // v_bar_j of 64 key blocks each) go through the same online softmax,
      // every block of the group taking the key blocks it did not keep.
      const __bf16* Kbs = p.kbar_bf + (size_t)bh * n_words * 64 * D;
      // value tiles: V^T order, or (LM) row-major, loaded like the K tiles
      const __bf16* Vbs = (LM ? p.vbar_bf : p.vbar_t) + (size_t)bh * n_words * D * 64;
      const int vb_off = LM ? dl.kc_off : dl.v_off;
      SOL_WAIT_VM();   // both buffers free: every load landed, every wave past its last tile
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      issue_tile<D>(sbufA, Kbs, dl.kc_off, 4096, Vbs, vb_off, 4096, dl);
#define SOL_VSTEP(CURB, NEXTB)                                                    \
      {                                                                           \
        const uint64_t pad = (c == n_words - 1 && (n_b & 63)) ? ~0ull << (n_b & 63) : 0ull; \
        SOL_WAIT_VM();                                                            \
        asm volatile("" ::: "memory");                                            \
        __builtin_amdgcn_s_barrier();                                             \
        asm volatile("" ::: "memory");                                            \
        if (c + 1 < n_words)                                                      \
          issue_tile<D>(NEXTB, Kbs + (size_t)(c + 1) * 64 * D, dl.kc_off, 4096, Vbs + (size_t)(c + 1) * D * 64, vb_off, 4096, dl); \
        _Pragma("unroll") for (int g = 0; g < kGMax; ++g) {                       \
          uint64_t ex = g < nG ? (masks[g * n_words + c] | pad) : ~0ull;          \
          ex = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ex >> 32)) << 32) | \
               (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ex);   /* uniform */ \
          if (ex != ~0ull) tile_bf16<D, true, kXO, LM>(sts[g], CURB, lofs, ex);   \
        }                                                                         \
        ++c;                                                                      \
      }
      int c = 0;
      while (true) {
        SOL_VSTEP(sbufA, sbufB)
        if (c >= n_words) break;
        SOL_VSTEP(sbufB, sbufA)
        if (c >= n_words) break;
      }
#undef SOL_VSTEP
    }
#undef SOL_STEP
#undef SOL_WAIT_VM
    // no LDS load may land after the workgroup has released its LDS
    __builtin_amdgcn_s_waitcnt(0xF70);
#pragma unroll
    for (int g = 0; g < kGMax; ++g)
      if (g < nG) epilogue<T, D>(sts[g], p, bh, qi0 + g, g, row, lane, qa, misc);
  } else {
    // fp32: the blocks one after another, one tile at a time
    ExactState<T, D> st;
    for (int g = 0; g < nG; ++g) {
      zero_state<T, D>(st);
      load_q<T, D>(st, Qh + ((long long)(qi0 + g) * kBlock + row) * p.qs.n, lane);
      for (int wi = 0; wi < n_words; ++wi) {
        uint64_t word = masks[g * n_words + wi];
        while (word) {
          const int j = wi * 64 + (int)__builtin_ctzll(word);
          word &= word - 1;
          __syncthreads();
          commit_f32<D>(reinterpret_cast<float*>(sbufA), reinterpret_cast<float*>(sbufA + Gm::kKBytes),
                        reinterpret_cast<const float*>(Kh), reinterpret_cast<const float*>(Vh), p.ks.n, p.vs.n, j, t);
          __syncthreads();
          tile_f32<D>(st, sbufA, lane);
        }
      }
      if constexpr (MODE == kModeCorrRow) {
        // per-row correction: tiles of block summaries (k_bar_j, v_bar_j) of
        // 64 key blocks each; kept blocks and blocks past n_b get no weight
        using Gm2 = Geom<float, D>;
        float* stK = reinterpret_cast<float*>(sbufA);
        float* stV = reinterpret_cast<float*>(sbufA + Gm2::kKBytes);
        for (int c = 0; c < n_words; ++c) {
          const uint64_t pad = (c == n_words - 1 && (n_b & 63)) ? ~0ull << (n_b & 63) : 0ull;
          const uint64_t ex = masks[g * n_words + c] | pad;
          if (ex == ~0ull) continue;   // uniform over the workgroup
          __syncthreads();
          for (int e = t; e < 64 * (D / 4); e += 256) {
            const int r = e / (D / 4), cc = e % (D / 4), jj = 64 * c + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (jj < n_b) {
              kx = reinterpret_cast<const float4*>(p.kbar + ((size_t)bh * n_b + jj) * D)[cc];
              vx = reinterpret_cast<const float4*>(p.vsum + ((size_t)bh * n_b + jj) * D)[cc];
            }
            const float sc = 1.0f / kBlock;   // v_bar = vsum / 64, exact
            *reinterpret_cast<float4*>(stK + r * Gm2::kKPitch + cc * 4) = kx;
            *reinterpret_cast<float4*>(stV + r * Gm2::kVPitch + cc * 4) =
                make_float4(vx.x * sc, vx.y * sc, vx.z * sc, vx.w * sc);
          }
          __syncthreads();
          tile_f32<D, true>(st, sbufA, lane, ex);
        }
      }
      epilogue<T, D>(st, p, bh, qi0 + g, g, row, lane, qa, misc);
    }
  }
  if (p.item_clock) {
    __syncthreads();   // every wave of the workgroup is done
    if (t == 0) {
      uint64_t* c = p.item_clock + 2 * ((size_t)bh * n_b + qi0);
      c[0] = clk0;
      c[1] = __builtin_amdgcn_s_memrealtime();
    }
  }
}

#ifdef SOL_FUSED_ROW_TU
}  // namespace

// This translation unit holds only the bf16 kernels of the per-row correction
// (built with the max-ILP scheduler, under which their register demand fits
// without spills; the other kernels run faster under the default one).
const void* fused_row_kernel_bf16(int d, bool low_memory) {
  if (low_memory)
    return d == 64 ? (const void*)fused_kernel<__bf16, 64, kModeCorrRow, true>
                   : (const void*)fused_kernel<__bf16, 128, kModeCorrRow, true>;
  return d == 64 ? (const void*)fused_kernel<__bf16, 64, kModeCorrRow>
                 : (const void*)fused_kernel<__bf16, 128, kModeCorrRow>;
}
const void* fused_row_reset_kernel() { return (const void*)queue_reset_kernel; }

}  // namespace sol
#else

// Queue slots of every fused launch of this library (all instantiations, both
// translation units' arrays), so that launches in flight together never share
// a slot.
QueueSlots g_queue_slots;

template <typename T, int D, bool LM>
const void* kernel_for_lm(const FusedArgs& a) {
  if (a.mask_in) return (const void*)fused_kernel<T, D, kModeGiven, LM>;
  if (a.correction_row) {
    if constexpr (std::is_same<T, __bf16>::value) return fused_row_kernel_bf16(D, LM);   // own translation unit
    else return (const void*)fused_kernel<T, D, kModeCorrRow>;
  }
  return a.correction ? (const void*)fused_kernel<T, D, kModeCorr, LM> : (const void*)fused_kernel<T, D, kModeRoute, LM>;
}
// the low-memory mode changes only the bf16 value tiles (fp32 stages V from the input)
template <typename T, int D>
const void* kernel_for(const FusedArgs& a) {
  if constexpr (std::is_same<T, __bf16>::value)
    if (a.low_memory) return kernel_for_lm<T, D, true>(a);
  return kernel_for_lm<T, D, false>(a);
}

template <typename T, int D>
hipError_t fused_impl(const Shape& s, const FusedArgs& a, hipStream_t st) {
  const FusedGeom g = fused_geom(s, std::is_same<T, __bf16>::value ? Dtype::BF16 : Dtype::F32);
  if (g.G < 1) return hipErrorInvalidValue;   // n_b too large for the LDS proxy rows
  FusedParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.out = a.out;
  p.vt = a.ws.vt;
  p.kbar_bf = a.ws.kbar_bf;
  p.vbar_t = a.ws.vbar_t;
  p.vbar_bf = a.ws.vbar_bf;
  p.kbar = a.ws.kbar;
  p.kbar_t = a.ws.kbar_t; p.vsum = a.ws.vsum; p.kmean = a.ws.kmean; p.kcov = a.ws.kcov;
  p.n_b = s.n_b; p.n_b_pad = s.n_b_pad; p.n_words = s.n_words;
  p.G = g.G; p.n_groups = g.n_groups; p.BH = s.BH(); p.per_xcd = g.per_xcd;
  p.N = s.N;
  p.H = s.H;
  p.qs = a.io.q; p.ks = a.io.k; p.vs = a.io.v; p.os = a.io.o;
  p.beta = a.beta; p.beta_mode = a.beta_mode;
  p.kept_per_row = a.kept_per_row; p.mask_bits = a.mask_bits; p.tau_out = a.tau;
  p.item_clock = a.item_clock;
  p.mask_in = a.mask_in;
  p.text_blocks = a.text_blocks;
  p.dyn_heads = g.dyn_heads;
  p.n_static_wg = g.n_static_wg;
  // a launch recorded into a graph keeps its slot for every replay: it takes
  // one from the range eager launches never use
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  hipError_t ec = hipStreamIsCapturing(st, &cap);
  if (ec != hipSuccess) return ec;
  p.qslot = g_queue_slots.take(cap != hipStreamCaptureStatusNone);
  const dim3 grid((unsigned)(g.n_static_wg + g.workers));
  // this launch's queue counter, zeroed by a kernel of the fused kernel's own
  // translation unit (a kernel rather than a memset, so that the launch
  // sequence can be captured in a graph)
  const bool row_tu = std::is_same<T, __bf16>::value && a.correction_row && !a.mask_in;
  const void* reset = row_tu ? fused_row_reset_kernel() : (const void*)queue_reset_kernel;
  int slot_arg = p.qslot;
  void* rargs[] = {&slot_arg};
  hipError_t e0 = hipLaunchKernel(reset, dim3(1), dim3(64), rargs, 0, st);
  if (e0 != hipSuccess) return e0;
  const void* fn = kernel_for<T, D>(a);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, g.lds_bytes);
  if (e != hipSuccess) return e;
  void* args[] = {&p};
  e = hipLaunchKernel(fn, grid, dim3(256), args, g.lds_bytes, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

template <typename T, int D>
FusedGeom geom_impl(const Shape& s) {
  using L = Lds<T, D>;
  FusedGeom g;
  const int cap = L::rows_per_buf(s.n_b_pad) * Geom<T, D>::kBuffers;   // proxy rows that fit
  g.G = cap < 1 ? 0 : (cap < kGMax ? cap : kGMax);
  g.n_groups = g.G ? (s.n_b + g.G - 1) / g.G : 0;
  g.items = s.BH() * g.n_groups;
  g.per_xcd = (g.n_groups + 7) / 8;
  // the last head's items are dealt from a queue by twice as many workers
  g.dyn_heads = s.BH() > 0 ? 1 : 0;
  g.n_static_wg = 8 * g.per_xcd * (s.BH() - g.dyn_heads);
  g.workers = 8 * ((2LL * g.dyn_heads * g.n_groups + 7) / 8);
  g.lds_bytes = L::bytes(g.G, s.n_words);
  return g;
}

}  // namespace

FusedGeom fused_geom(const Shape& s, Dtype dt) {
  if (dt == Dtype::BF16) return s.d == 64 ? geom_impl<__bf16, 64>(s) : geom_impl<__bf16, 128>(s);
  return s.d == 64 ? geom_impl<float, 64>(s) : geom_impl<float, 128>(s);
}

hipError_t launch_fused(const Shape& s, Dtype dt, const FusedArgs& a, hipStream_t stream) {
  if (dt == Dtype::BF16)
    return s.d == 64 ? fused_impl<__bf16, 64>(s, a, stream) : fused_impl<__bf16, 128>(s, a, stream);
  return s.d == 64 ? fused_impl<float, 64>(s, a, stream) : fused_impl<float, 128>(s, a, stream);
}

}  // namespace sol
#endif
