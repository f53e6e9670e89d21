// C-ABI host runtime of the Sol-Attn library: argument validation (before any
// device call), workspace layout, the library-owned workspace of sol_attn_fwd,
// HIP error -> sol_status mapping and the per-thread error message.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "../../include/sol_attn.h"
#include "sol_internal.hpp"

namespace sol {

static size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

Layout make_layout(const Shape& s) {
  const size_t bh = (size_t)s.BH(), d = (size_t)s.d, nb = (size_t)s.n_b;
  Layout L;
  size_t off = 0;
  L.kbar_t = off;   off += up256(bh * d * (size_t)s.n_b_pad * 4);
  L.kbar = off;     off += up256(bh * nb * d * 4);
  L.vsum = off;     off += up256(bh * nb * d * 4);
  L.kmean = off;    off += up256(bh * d * 4);
  L.kcov = off;     off += up256(bh * d * d * 4);
  L.qbar = off;     off += up256(bh * nb * d * 4);
  L.kbar_bf = off;  off += up256(bh * (size_t)s.n_words * 64 * d * 2);
  L.vbar_t = off;   off += up256(bh * (size_t)s.n_words * 64 * d * 2);
  L.vbar_bf = off;  off += up256(bh * (size_t)s.n_words * 64 * d * 2);
  L.s1_part = off;  off += up256(bh * (size_t)s.cov_parts * d * 8);
  L.s2_part = off;  off += up256(bh * (size_t)s.cov_parts * d * d * 8);
  L.vt = off;       off += up256(bh * nb * d * 64 * 2);
  L.total = off;
  return L;
}

Workspace bind_workspace(const Shape& s, void* base) {
  const Layout L = make_layout(s);
  char* b = static_cast<char*>(base);
  Workspace w;
  w.kbar_t = reinterpret_cast<float*>(b + L.kbar_t);
  w.kbar = reinterpret_cast<float*>(b + L.kbar);
  w.vsum = reinterpret_cast<float*>(b + L.vsum);
  w.kmean = reinterpret_cast<float*>(b + L.kmean);
  w.kcov = reinterpret_cast<float*>(b + L.kcov);
  w.vt = reinterpret_cast<__bf16*>(b + L.vt);
  w.qbar = reinterpret_cast<float*>(b + L.qbar);
  w.kbar_bf = reinterpret_cast<__bf16*>(b + L.kbar_bf);
  w.vbar_t = reinterpret_cast<__bf16*>(b + L.vbar_t);
  w.vbar_bf = reinterpret_cast<__bf16*>(b + L.vbar_bf);
  w.s1_part = reinterpret_cast<double*>(b + L.s1_part);
  w.s2_part = reinterpret_cast<double*>(b + L.s2_part);
  return w;
}

}  // namespace sol

namespace {

thread_local char g_err[512] = "";

sol_status fail(sol_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sol_status ok() {
  g_err[0] = '\0';
  return SOL_OK;
}

sol_status device_fail(hipError_t e, const char* what) {
  return fail(SOL_ERR_DEVICE, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Shape checks shared by every entry point; fills `s` on success.
sol_status check_shape(int B, int H, int N, int d, sol::Shape* s) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0)
    return fail(SOL_ERR_INVALID_ARG, "B, H, N, d must be positive (got %d, %d, %d, %d)", B, H, N, d);
  if (N % sol::kBlock != 0)
    return fail(SOL_ERR_INVALID_ARG, "N = %d is not a multiple of the 64-token block", N);
  if (d != 64 && d != 128)
    return fail(SOL_ERR_UNSUPPORTED, "head dim d = %d is not supported (64 or 128)", d);
  if (N / sol::kBlock > sol::kMaxBlocks)
    return fail(SOL_ERR_UNSUPPORTED, "N = %d exceeds the supported maximum %d", N,
                sol::kMaxBlocks * sol::kBlock);
  if ((long long)B * H > 65535)
    return fail(SOL_ERR_UNSUPPORTED, "B*H = %lld exceeds 65535", (long long)B * H);
  s->B = B; s->H = H; s->N = N; s->d = d;
  s->n_b = N / sol::kBlock;
  s->n_b_pad = (s->n_b + 3) & ~3;
  s->n_words = (s->n_b + 63) / 64;
  // partials of 128 key blocks, halved (down to 32) while the moment kernel
  // would get fewer than 512 workgroups; this keeps B*H*cov_parts <= 512
  // whenever the chunk shrinks, so the partials stay bounded
  s->cov_chunk = sol::kCovChunk;
  while (s->cov_chunk > 32 && 2LL * B * H * ((s->n_b + s->cov_chunk - 1) / s->cov_chunk) < 512)
    s->cov_chunk /= 2;
  s->cov_parts = (s->n_b + s->cov_chunk - 1) / s->cov_chunk;
  if ((long long)B * H * s->n_b > 0x7fffffffLL)
    return fail(SOL_ERR_UNSUPPORTED, "B*H*N/64 exceeds the launch grid limit");
  return SOL_OK;
}

sol_status check_flags(unsigned flags) {
  if (flags & ~SOL_FLAGS_ALL) return fail(SOL_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~SOL_FLAGS_ALL);
  return SOL_OK;
}

// Device pointers the kernels read or write with 16-byte vector accesses
// (q, k, v, out), the workspace (arrays at 256-byte offsets, read as float4
// and double) and the debug outputs (natural alignment of their elements).
sol_status check_align(const void* p, size_t a, const char* name) {
  if (p && reinterpret_cast<uintptr_t>(p) % a)
    return fail(SOL_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, a);
  return SOL_OK;
}

sol_status check_io_align(const void* q, const void* k, const void* v, const void* out) {
  sol_status st;
  if (q && (st = check_align(q, 16, "q")) != SOL_OK) return st;
  if ((st = check_align(k, 16, "k")) != SOL_OK) return st;
  if ((st = check_align(v, 16, "v")) != SOL_OK) return st;
  if (out && (st = check_align(out, 16, "out")) != SOL_OK) return st;
  return SOL_OK;
}

sol_status check_dbg_align(const sol_debug* dbg) {
  if (!dbg) return SOL_OK;
  sol_status st;
  if ((st = check_align(dbg->kept_per_row, 4, "kept_per_row")) != SOL_OK) return st;
  if ((st = check_align(dbg->mask_bits, 8, "mask_bits")) != SOL_OK) return st;
  if ((st = check_align(dbg->tau, 4, "tau")) != SOL_OK) return st;
  return check_align(dbg->item_clock, 8, "item_clock");
}

// Workspace bytes of a shape: the whole layout, or with SOL_LOW_MEMORY the
// part before the V^T copy (the last array).
size_t ws_need(const sol::Shape& s, unsigned flags) {
  const sol::Layout L = sol::make_layout(s);
  return (flags & SOL_LOW_MEMORY) ? L.vt : L.total;
}

// A caller workspace: present, large enough for the shape and mode, 256-byte aligned.
sol_status check_workspace(const sol::Shape& s, const void* ws, size_t ws_bytes, unsigned flags) {
  const size_t need = ws_need(s, flags);
  if (!ws || ws_bytes < need)
    return fail(SOL_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu%s)", need, ws_bytes, ws ? "" : ", NULL");
  return check_align(ws, 256, "workspace");
}

sol::Dtype dtype_of(unsigned flags) { return (flags & SOL_F32) ? sol::Dtype::F32 : sol::Dtype::BF16; }

sol_status finish(unsigned flags, hipStream_t st) {
  if (flags & SOL_SYNC) {
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return device_fail(e, "hipStreamSynchronize");
  }
  return ok();
}

sol_status summaries_checked(const sol::Shape& s, const void* k, const void* v, unsigned flags,
                             void* ws, hipStream_t st, const sol::IoStrides* io = nullptr) {
  const sol::Workspace w = sol::bind_workspace(s, ws);
  const sol::IoStrides x = io ? *io : sol::contiguous_io(s);
  hipError_t e = sol::launch_prepass(s, dtype_of(flags), k, v, x.k, x.v, w, !(flags & SOL_LOW_MEMORY), st);
  if (e != hipSuccess) return device_fail(e, "block-summary pre-pass launch");
  return SOL_OK;
}

sol_status fused_checked(const sol::Shape& s, const void* q, const void* k, const void* v, void* out,
                         float beta, unsigned flags, const void* ws, const sol_debug* dbg,
                         hipStream_t st, int text_blocks = 0, const sol::IoStrides* io = nullptr) {
  sol::FusedArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.ws = sol::bind_workspace(s, const_cast<void*>(ws));
  a.beta = beta;
  a.beta_mode = (flags & SOL_DENSE) || beta == -INFINITY ? sol::kBetaMinusInf
                : beta == INFINITY                       ? sol::kBetaPlusInf
                                                         : sol::kBetaFinite;
  a.correction = (flags & (SOL_CORRECTION | SOL_CORRECTION_ROW)) != 0;
  a.correction_row = (flags & SOL_CORRECTION_ROW) != 0;
  a.kept_per_row = dbg ? dbg->kept_per_row : nullptr;
  a.mask_bits = dbg ? dbg->mask_bits : nullptr;
  a.tau = dbg ? dbg->tau : nullptr;
  a.item_clock = dbg ? dbg->item_clock : nullptr;
  a.mask_in = nullptr;
  a.text_blocks = text_blocks;
  a.io = io ? *io : sol::contiguous_io(s);
  a.low_memory = (flags & SOL_LOW_MEMORY) != 0;
  hipError_t e = sol::launch_fused(s, dtype_of(flags), a, st);
  if (e != hipSuccess) return device_fail(e, "fused kernel launch");
  return SOL_OK;
}

sol_status check_fused_args(const void* q, const void* k, const void* v, void* out, float beta,
                            unsigned flags) {
  if (!q || !k || !v || !out) return fail(SOL_ERR_INVALID_ARG, "q, k, v and out must be non-null");
  if (isnan(beta)) return fail(SOL_ERR_INVALID_ARG, "beta is NaN");
  sol_status st = check_flags(flags);
  if (st != SOL_OK) return st;
  return check_io_align(q, k, v, out);
}

// Strides of one tensor from the caller (NULL: contiguous), validated.
sol_status take_strides(const sol::Shape& s, unsigned flags, const sol_strides* in, const void* ptr,
                        const char* name, bool is_out, sol::TStrides* st) {
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(SOL_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  if (!in) {
    *st = sol::contiguous_strides(s);
    return SOL_OK;
  }
  const long long unit = (flags & SOL_F32) ? 4 : 8;   // elements per 16 bytes
  const long long v[3] = {in->b, in->h, in->n};
  const int ext[3] = {s.B, s.H, s.N};
  const char* dim[3] = {"b", "h", "n"};
  for (int i = 0; i < 3; ++i) {
    if (v[i] < 0 || (v[i] == 0 && ext[i] > 1))
      return fail(SOL_ERR_INVALID_ARG, "%s stride %s must be positive (got %lld)", name, dim[i], v[i]);
    if (v[i] % unit)
      return fail(SOL_ERR_INVALID_ARG, "%s stride %s must be a multiple of %lld elements (got %lld)", name,
                  dim[i], unit, v[i]);
  }
  if (in->n >= (1ll << 24)) return fail(SOL_ERR_INVALID_ARG, "%s stride n must be below 2^24", name);
  if (is_out && in->n < s.d) return fail(SOL_ERR_INVALID_ARG, "%s stride n must be at least d", name);
  *st = sol::TStrides{in->b, in->h, in->n};
  return SOL_OK;
}

// Library-owned workspace of sol_attn_fwd, one per device.
struct OwnedWorkspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
// Held until the process ends (no hipFree from static destructors, which may
// run after the HIP runtime has shut down).
std::mutex g_ws_mutex;
std::vector<OwnedWorkspace> g_ws;

}  // namespace

extern "C" {

int sol_abi_version(void) { return SOL_ATTN_ABI_VERSION; }

const char* sol_last_error(void) { return g_err; }

size_t sol_attn_workspace_bytes(int B, int H, int N, int d) {
  sol::Shape s;
  char saved[sizeof(g_err)];
  memcpy(saved, g_err, sizeof(g_err));
  const sol_status st = check_shape(B, H, N, d, &s);
  memcpy(g_err, saved, sizeof(g_err));
  return st == SOL_OK ? sol::make_layout(s).total : 0;
}

size_t sol_attn_workspace_bytes_flags(int B, int H, int N, int d, unsigned flags) {
  sol::Shape s;
  char saved[sizeof(g_err)];
  memcpy(saved, g_err, sizeof(g_err));
  const sol_status st = check_shape(B, H, N, d, &s);
  memcpy(g_err, saved, sizeof(g_err));
  return st == SOL_OK ? ws_need(s, flags) : 0;
}

sol_status sol_attn_workspace_layout(int B, int H, int N, int d, sol_workspace_layout* layout) {
  if (!layout) return fail(SOL_ERR_INVALID_ARG, "layout must be non-null");
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  const sol::Layout L = sol::make_layout(s);
  layout->total_bytes = L.total;
  layout->kbar_t = L.kbar_t;
  layout->kbar = L.kbar;
  layout->vsum = L.vsum;
  layout->kmean = L.kmean;
  layout->kcov = L.kcov;
  layout->vt = L.vt;
  layout->qbar = L.qbar;
  layout->kbar_bf = L.kbar_bf;
  layout->vbar_t = L.vbar_t;
  layout->scratch = L.s1_part;
  layout->vbar_bf = L.vbar_bf;
  return ok();
}

sol_status sol_block_summaries(const void* k, const void* v, int B, int H, int N, int d,
                               unsigned flags, void* workspace, size_t ws_bytes, void* hip_stream) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if (!k || !v) return fail(SOL_ERR_INVALID_ARG, "k and v must be non-null");
  if ((st = check_flags(flags)) != SOL_OK) return st;
  if ((st = check_io_align(nullptr, k, v, nullptr)) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = summaries_checked(s, k, v, flags, workspace, str)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_fused(const void* q, const void* k, const void* v, void* out, int B, int H,
                          int N, int d, float beta, unsigned flags, const void* workspace,
                          size_t ws_bytes, const sol_debug* dbg, void* hip_stream) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  if ((st = check_dbg_align(dbg)) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = fused_checked(s, q, k, v, out, beta, flags, workspace, dbg, str)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_masked(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int N, int d, const uint64_t* mask_bits, unsigned flags,
                           const void* workspace, size_t ws_bytes, int32_t* kept_per_row,
                           void* hip_stream) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if (!q || !k || !v || !out || !mask_bits)
    return fail(SOL_ERR_INVALID_ARG, "q, k, v, out and mask_bits must be non-null");
  if ((st = check_flags(flags)) != SOL_OK) return st;
  if (flags & (SOL_CORRECTION | SOL_CORRECTION_ROW | SOL_DENSE))
    return fail(SOL_ERR_INVALID_ARG, "the given-mask mode takes neither SOL_CORRECTION(_ROW) nor SOL_DENSE");
  if ((st = check_io_align(q, k, v, out)) != SOL_OK) return st;
  if ((st = check_align(mask_bits, 8, "mask_bits")) != SOL_OK) return st;
  if ((st = check_align(kept_per_row, 4, "kept_per_row")) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  sol::FusedArgs a;
  a.q = q; a.k = k; a.v = v; a.out = out;
  a.ws = sol::bind_workspace(s, const_cast<void*>(workspace));
  a.beta = 0.f;
  a.beta_mode = sol::kBetaFinite;
  a.correction = false;
  a.correction_row = false;
  a.kept_per_row = kept_per_row;
  a.mask_bits = nullptr;
  a.tau = nullptr;
  a.item_clock = nullptr;
  a.mask_in = mask_bits;
  a.text_blocks = 0;
  a.io = sol::contiguous_io(s);
  a.low_memory = (flags & SOL_LOW_MEMORY) != 0;
  hipError_t e = sol::launch_fused(s, dtype_of(flags), a, str);
  if (e != hipSuccess) return device_fail(e, "given-mask kernel launch");
  return finish(flags, str);
}

sol_status sol_route(const void* q, int B, int H, int N, int d, unsigned flags, int mode,
                     float beta, int topk, float topp, const void* workspace, size_t ws_bytes,
                     float* proxy_map, uint64_t* mask_bits, int32_t* kept_per_row,
                     int32_t* topk_idx, void* hip_stream) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if (!q || !proxy_map || !mask_bits)
    return fail(SOL_ERR_INVALID_ARG, "q, proxy_map and mask_bits must be non-null");
  if ((st = check_flags(flags)) != SOL_OK) return st;
  if (flags & (SOL_CORRECTION | SOL_CORRECTION_ROW | SOL_DENSE))
    return fail(SOL_ERR_INVALID_ARG, "routing takes neither SOL_CORRECTION(_ROW) nor SOL_DENSE");
  if (mode != SOL_ROUTE_THRESHOLD && mode != SOL_ROUTE_TOPK && mode != SOL_ROUTE_TOPP)
    return fail(SOL_ERR_INVALID_ARG, "unknown routing mode %d", mode);
  if (mode == SOL_ROUTE_THRESHOLD && isnan(beta)) return fail(SOL_ERR_INVALID_ARG, "beta is NaN");
  if (mode == SOL_ROUTE_TOPP && !(topp == topp)) return fail(SOL_ERR_INVALID_ARG, "top_p is NaN");
  if (mode == SOL_ROUTE_TOPK && topk < 0) return fail(SOL_ERR_INVALID_ARG, "top_k is negative");
  if ((st = check_align(q, 16, "q")) != SOL_OK) return st;
  if ((st = check_align(proxy_map, 4, "proxy_map")) != SOL_OK) return st;
  if ((st = check_align(mask_bits, 8, "mask_bits")) != SOL_OK) return st;
  if ((st = check_align(kept_per_row, 4, "kept_per_row")) != SOL_OK) return st;
  if ((st = check_align(topk_idx, 4, "topk_idx")) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  sol::RouteArgs a;
  a.q = q;
  a.qs = sol::contiguous_strides(s);
  a.ws = sol::bind_workspace(s, const_cast<void*>(workspace));
  a.mode = mode;
  a.beta = beta;
  a.beta_mode = beta == -INFINITY ? sol::kBetaMinusInf : beta == INFINITY ? sol::kBetaPlusInf : sol::kBetaFinite;
  a.topk = topk;
  a.topp = topp;
  a.proxy_map = proxy_map;
  a.mask = mask_bits;
  a.kept = kept_per_row;
  a.idx = mode == SOL_ROUTE_TOPK ? topk_idx : nullptr;
  hipError_t e = sol::launch_route(s, dtype_of(flags), a, str);
  if (e != hipSuccess) return device_fail(e, "routing launch");
  return finish(flags, str);
}

sol_status sol_attn_fused_joint(const void* q, const void* k, const void* v, void* out, int B,
                                int H, int N, int d, float beta, unsigned flags, int text_blocks,
                                const void* workspace, size_t ws_bytes, const sol_debug* dbg,
                                void* hip_stream) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  if (text_blocks < 0 || text_blocks > s.n_b)
    return fail(SOL_ERR_INVALID_ARG, "text_blocks must be in [0, n_b] (got %d, n_b %d)", text_blocks, s.n_b);
  if ((st = check_dbg_align(dbg)) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = fused_checked(s, q, k, v, out, beta, flags, workspace, dbg, str, text_blocks)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H,
                           int N, int d, float beta, unsigned flags, void* hip_stream,
                           void* workspace, size_t ws_bytes, const sol_debug* dbg) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  if ((st = check_dbg_align(dbg)) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = summaries_checked(s, k, v, flags, workspace, str)) != SOL_OK) return st;
  if ((st = fused_checked(s, q, k, v, out, beta, flags, workspace, dbg, str)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_fwd_strided(const void* q, const void* k, const void* v, void* out, int B, int H,
                                int N, int d, const sol_strides* q_strides, const sol_strides* k_strides,
                                const sol_strides* v_strides, const sol_strides* out_strides, float beta,
                                unsigned flags, void* hip_stream, void* workspace, size_t ws_bytes,
                                const sol_debug* dbg) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  sol::IoStrides io;
  if ((st = take_strides(s, flags, q_strides, q, "q", false, &io.q)) != SOL_OK) return st;
  if ((st = take_strides(s, flags, k_strides, k, "k", false, &io.k)) != SOL_OK) return st;
  if ((st = take_strides(s, flags, v_strides, v, "v", false, &io.v)) != SOL_OK) return st;
  if ((st = take_strides(s, flags, out_strides, out, "out", true, &io.o)) != SOL_OK) return st;
  if ((st = check_dbg_align(dbg)) != SOL_OK) return st;
  if ((st = check_workspace(s, workspace, ws_bytes, flags)) != SOL_OK) return st;
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = summaries_checked(s, k, v, flags, workspace, str, &io)) != SOL_OK) return st;
  if ((st = fused_checked(s, q, k, v, out, beta, flags, workspace, dbg, str, 0, &io)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                                int N, int d, float beta, unsigned flags, void* hip_stream,
                                const sol_debug* dbg) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  if ((st = check_dbg_align(dbg)) != SOL_OK) return st;
  const size_t need = ws_need(s, flags);
  if (need > sol::kNoAllocScratchBytes)
    return fail(SOL_ERR_UNSUPPORTED, "the shape needs %zu bytes of scratch, above the %zu-byte maximum of "
                "sol_attn_fwd_noalloc (use sol_attn_fwd_ex with a workspace)", need, sol::kNoAllocScratchBytes);
  void* ws = nullptr;
  hipError_t e = sol::noalloc_scratch(&ws);
  if (e != hipSuccess) return device_fail(e, "scratch address lookup");
  hipStream_t str = static_cast<hipStream_t>(hip_stream);
  if ((st = summaries_checked(s, k, v, flags, ws, str)) != SOL_OK) return st;
  if ((st = fused_checked(s, q, k, v, out, beta, flags, ws, dbg, str)) != SOL_OK) return st;
  return finish(flags, str);
}

sol_status sol_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int N,
                        int d, float beta, unsigned flags) {
  sol::Shape s;
  sol_status st = check_shape(B, H, N, d, &s);
  if (st != SOL_OK) return st;
  if ((st = check_fused_args(q, k, v, out, beta, flags)) != SOL_OK) return st;
  const size_t need = ws_need(s, flags);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  if ((size_t)dev >= g_ws.size()) g_ws.resize(dev + 1);
  OwnedWorkspace& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr) {
      // the previous workspace may still be read by queued work on any stream
      if ((e = hipDeviceSynchronize()) != hipSuccess) return device_fail(e, "hipDeviceSynchronize");
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, need) != hipSuccess) {
      w.ptr = nullptr;
      (void)hipGetLastError();
      return fail(SOL_ERR_NOMEM, "could not allocate a %zu-byte workspace", need);
    }
    w.bytes = need;
  }
  if ((st = summaries_checked(s, k, v, flags, w.ptr, nullptr)) != SOL_OK) return st;
  if ((st = fused_checked(s, q, k, v, out, beta, flags, w.ptr, nullptr, nullptr)) != SOL_OK) return st;
  return finish(flags, nullptr);
}

}  // extern "C"
