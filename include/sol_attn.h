/*
 * sol_attn.h - C ABI of the Sol-Attn forward library for AMD MI355X (gfx950).
 *
 * What it computes (per batch b, head h, 64-token query block i):
 *   q_bar_i, k_bar_j, v_bar_j : means over each block of 64 tokens;
 *   s_hat_ij = q_bar_i . k_bar_j / sqrt(d)            (block proxy score);
 *   tau_i    = mu_i + beta * sigma_i, with mu_i and sigma_i the mean and
 *              population std of row i of s_hat, obtained in closed form from
 *              the mean m and the centred covariance C of the key summaries:
 *              mu_i = q_bar_i.m / sqrt(d), sigma_i^2 = q_bar_i^T C q_bar_i / d;
 *   S_i      = { j : s_hat_ij > tau_i } (strict);
 *   out_r    = softmax attention of query row r over the tokens of the blocks
 *              in S_i, plus (with SOL_CORRECTION) every block j outside S_i
 *              entered as 64 virtual tokens of logit s_hat_ij and value v_bar_j.
 * Sources: page "Sol-Attn: l'attenzione sparsa che sceglie al volo, per
 * generare video piu in fretta" (paithon.it), sections "Perche l'attenzione
 * pesa tanto nei video" (64-token blocks, mean-pooled proxy), "Una soglia per
 * ogni riga" (threshold equation; closed-form mu/sigma from the key-summary
 * mean and d x d second moments) and "Scegliere mentre si calcola" (in-pass
 * test against tau_i; excluded blocks reused as zeroth-order terms in the
 * same online-softmax state); the paper abstract (routing, sparse compute and
 * correction in one online-softmax pass). The 1/sqrt(d) proxy scale and the
 * exact virtual-token form are this library's reading of those passages.
 *
 * Tensor layout: q, k, v, out are contiguous [B][H][N][d] arrays in device
 * memory, all of one dtype (bfloat16 by default, float32 with SOL_F32);
 * sol_attn_fwd_strided also takes other strides (e.g. [B][N][H][d]).
 * N must be a multiple of 64 (no partial block), 64 <= N <= 262144, and
 * d must be 64 or 128. Softmax scale is 1/sqrt(d).
 *
 * Ownership: every pointer is owned by the caller. The library keeps no
 * pointer after a call returns. Calls are asynchronous on the given HIP stream
 * (NULL = the null stream): buffers must stay alive until that stream has
 * finished the work. Nothing here allocates device memory except
 * sol_attn_fwd, which keeps one library-owned workspace per device. The fused
 * pass deals part of its work from a counter in the library's static device
 * memory (16 KB per device). Eager launches take one of 3072 counters
 * round-robin: on one stream any number of launches may be queued; across
 * streams, at most 3072 eager fused launches may be enqueued and not yet
 * finished at a time. A fused launch recorded into a graph keeps its counter
 * for every replay (the counter is cleared by a kernel of the graph); it takes
 * one of the other 1024 counters, round-robin, which eager launches never use.
 * So a graph must not be replayed concurrently with itself, nor with a graph
 * captured 1024 fused launches earlier or later.
 *
 * Alignment: q, k, v and out must be 16-byte aligned device pointers, a
 * caller workspace 256-byte aligned, and the optional int32 / float / uint64
 * outputs aligned to their element size; a misaligned pointer gives
 * SOL_ERR_INVALID_ARG.
 *
 * Errors: every entry point returns a sol_status and never aborts or throws.
 * Arguments are validated before any device call; on failure nothing has been
 * enqueued. sol_last_error() gives a message for the last failing call on the
 * calling thread.
 */
#ifndef SOL_ATTN_H
#define SOL_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SOL_ATTN_ABI_VERSION 4

typedef enum sol_status {
  SOL_OK = 0,
  SOL_ERR_INVALID_ARG = 1,   /* null pointer, size <= 0, N % 64 != 0, beta NaN, bad flags */
  SOL_ERR_UNSUPPORTED = 2,   /* d not in {64, 128}, N beyond the supported maximum       */
  SOL_ERR_DEVICE = 3,        /* a HIP call failed (message names it)                     */
  SOL_ERR_NOMEM = 4,         /* the library-owned workspace could not be allocated       */
  SOL_ERR_WORKSPACE = 5      /* caller workspace NULL or smaller than required           */
} sol_status;

/* flags (bitwise or) */
#define SOL_BF16       0x0u  /* q, k, v, out are bfloat16 (default)                         */
#define SOL_F32        0x1u  /* q, k, v, out are float32                                    */
#define SOL_CORRECTION 0x2u  /* fold every unselected block in as 64 virtual tokens         */
#define SOL_DENSE      0x4u  /* keep every block (same selection as beta = -INFINITY)       */
#define SOL_SYNC       0x8u  /* synchronise the stream before returning, report its errors  */
#define SOL_CORRECTION_ROW 0x10u /* correction with the per-row logit q_r . k_bar_j / sqrt(d)
                                    of every virtual token, instead of the block proxy
                                    s_hat_ij (implies SOL_CORRECTION)                         */
#define SOL_LOW_MEMORY 0x20u /* bf16: no V^T copy in the workspace; the fused pass reads
                                the value tiles from V itself (transposing LDS reads).
                                A smaller workspace (sol_attn_workspace_bytes_flags); the
                                same results bit for bit, some time more. Pass it to the
                                pre-pass and to the fused pass alike: a workspace whose
                                pre-pass ran with it holds no V^T for a pass without it,
                                and one whose pre-pass ran without it holds no row-major
                                v_bar tiles for a per-row-correction pass with it. Neither
                                mismatch is detected. No effect for float32 inputs.        */
#define SOL_FLAGS_ALL  0x3Fu

/* Optional per-call outputs, all device pointers owned by the caller, each may be NULL.
 * n_b = N / 64, W = ceil(n_b / 64).
 *   kept_per_row [B*H*n_b]      int32: |S_i| for each query block (row of blocks)
 *   mask_bits    [B*H*n_b*W]    uint64: bit (j % 64) of word j / 64 is set iff j in S_i
 *   tau          [B*H*n_b]      float: tau_i as used by the selection (-inf / +inf allowed)
 *   item_clock   [B*H*n_b][2]   uint64: for the workgroup whose first query block is i of
 *                               head (b, h), entry (b*H + h)*n_b + i holds the device's
 *                               100 MHz constant clock (s_memrealtime) when the workgroup
 *                               started and when its last wave finished; entries of query
 *                               blocks that start no workgroup are left untouched (a
 *                               workgroup takes up to 4 consecutive query blocks) */
typedef struct sol_debug {
  int32_t*  kept_per_row;
  uint64_t* mask_bits;
  float*    tau;
  uint64_t* item_clock;
} sol_debug;

/* Byte offsets, inside a workspace, of the arrays the block-summary pre-pass
 * writes (all float32 unless noted; BH = B*H; nbp = n_b rounded up to 4):
 *   kbar_t  [BH][d][nbp]  block-mean keys, transposed (k_bar_j[c] at [c][j])
 *   kbar    [BH][n_b][d]  block-mean keys
 *   vsum    [BH][n_b][d]  block sums of values (= 64 * v_bar_j)
 *   kmean   [BH][d]       m = mean over j of k_bar_j
 *   kcov    [BH][d][d]    C = (1/n_b) sum_j (k_bar_j - m)(k_bar_j - m)^T
 *   qbar    [BH][n_b][d]  block-mean queries, written by sol_route only
 *   kbar_bf [BH][W][64][d] bfloat16: k_bar_j of key blocks 64c .. 64c+63 as
 *                         tile c (zero past n_b), for SOL_CORRECTION_ROW
 *   vbar_t  [BH][W][d][64] bfloat16: v_bar_j of the same blocks, transposed,
 *                         columns in the vt key order (zero past n_b)
 *   vbar_bf [BH][W][64][d] bfloat16: v_bar_j of the same blocks, row-major
 *                         (zero past n_b) (these three written by the pre-pass
 *                         for bf16 inputs, vbar_bf with SOL_LOW_MEMORY only)
 *   scratch .. vt         scratch of the pre-pass
 *   vt      [BH][n_b][d][64] bfloat16, the last array: each 64 x d block of V
 *                         transposed, column c holding key 32*(c/32) + 4*g + s
 *                         for s = c%8 < 4, else 32*(c/32) + 16 + 4*g + s - 4,
 *                         with g = (c%32)/8 (written for bf16 inputs unless
 *                         SOL_LOW_MEMORY; a SOL_LOW_MEMORY workspace ends here,
 *                         its size is the vt offset) */
typedef struct sol_workspace_layout {
  size_t total_bytes;
  size_t kbar_t;
  size_t kbar;
  size_t vsum;
  size_t kmean;
  size_t kcov;
  size_t vt;
  size_t qbar;
  size_t kbar_bf;
  size_t vbar_t;
  size_t scratch;
  size_t vbar_bf;
} sol_workspace_layout;

/* ABI version of the loaded library (SOL_ATTN_ABI_VERSION it was built with). */
int sol_abi_version(void);

/* Message for the last non-OK status returned on this thread ("" if none).
 * Valid until the next library call on the same thread. */
const char* sol_last_error(void);

/* Workspace size in bytes for a problem, 0 if the shape is invalid or unsupported. */
size_t sol_attn_workspace_bytes(int B, int H, int N, int d);

/* The same for the calls' flags: with SOL_LOW_MEMORY, the bytes before the V^T
 * copy (vt offset); otherwise sol_attn_workspace_bytes. */
size_t sol_attn_workspace_bytes_flags(int B, int H, int N, int d, unsigned flags);

/* Offsets of the pre-pass arrays inside the workspace (see sol_workspace_layout). */
sol_status sol_attn_workspace_layout(int B, int H, int N, int d, sol_workspace_layout* layout);

/* Block-summary pre-pass: reads k and v once and writes k_bar, v sums, m and C
 * into `workspace` (layout above). Source of m and C: page "Sol-Attn:
 * l'attenzione sparsa che sceglie al volo" (paithon.it), section "Una soglia
 * per ogni riga", last paragraph (mean of the compressed keys and their d x d
 * second-moment matrix). flags: SOL_F32 selects the dtype, SOL_LOW_MEMORY
 * leaves out the V^T copy; other bits ignored. workspace: device memory of at
 * least sol_attn_workspace_bytes_flags(B, H, N, d, flags) bytes. */
sol_status sol_block_summaries(const void* k, const void* v, int B, int H, int N, int d,
                               unsigned flags, void* workspace, size_t ws_bytes,
                               void* hip_stream);

/* Fused pass: per query block, closed-form tau_i, in-pass proxy test of every
 * key block, exact attention on the kept blocks and (SOL_CORRECTION) the
 * virtual-token fold of the others, in one online-softmax state; writes out.
 * Source: same page, section "Scegliere mentre si calcola". `workspace` must
 * hold the pre-pass results of the same k, v and shape (it is only read).
 * dbg may be NULL. beta = -INFINITY or SOL_DENSE keeps every block;
 * beta = +INFINITY keeps none. */
sol_status sol_attn_fused(const void* q, const void* k, const void* v, void* out,
                          int B, int H, int N, int d, float beta, unsigned flags,
                          const void* workspace, size_t ws_bytes, const sol_debug* dbg,
                          void* hip_stream);

/* The fused pass for joint attention with a text segment: the last text_blocks
 * blocks of the sequence are text tokens, which are always computed exactly
 * (page "Sol-Attn: l'attenzione sparsa che sceglie al volo" (paithon.it),
 * section "Dove leggere con attenzione": the evaluated systems compute text
 * tokens exactly). The selection runs as in sol_attn_fused over all n_b key
 * blocks; then every query block also keeps the text key blocks, and a text
 * query block keeps every key block (a dense row). The caller pads the text
 * segment to whole 64-token blocks. text_blocks in [0, n_b], else
 * SOL_ERR_INVALID_ARG; 0 is sol_attn_fused. Other arguments as sol_attn_fused. */
sol_status sol_attn_fused_joint(const void* q, const void* k, const void* v, void* out,
                                int B, int H, int N, int d, float beta, unsigned flags,
                                int text_blocks, const void* workspace, size_t ws_bytes,
                                const sol_debug* dbg, void* hip_stream);

/* Block-sparse attention on a caller-given selection: no routing and no
 * correction, the same exact-attention pass as sol_attn_fused on the same
 * blocks. It is the plain block-sparse kernel the fused pass is measured
 * against (page "Sol-Attn: l'attenzione sparsa che sceglie al volo"
 * (paithon.it), section "I numeri": the fused kernel against a plain
 * block-sparse kernel on the same blocks). Needs the pre-pass workspace of
 * the same K, V (sol_block_summaries).
 *   mask_bits    [B*H*n_b*W] uint64, device, same layout as sol_debug.mask_bits:
 *                bit (j % 64) of word j / 64 of query block i keeps key block j;
 *                bits past n_b are ignored. A query block with no bit set gets
 *                zero output rows.
 *   kept_per_row [B*H*n_b] int32, device, optional (NULL): popcount of each row.
 * flags: SOL_F32, SOL_SYNC and SOL_LOW_MEMORY (as on the pre-pass that filled
 * the workspace); SOL_CORRECTION, SOL_CORRECTION_ROW or SOL_DENSE give
 * SOL_ERR_INVALID_ARG. Asynchronous on hip_stream like sol_attn_fused. */
sol_status sol_attn_masked(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int N, int d, const uint64_t* mask_bits,
                           unsigned flags, const void* workspace, size_t ws_bytes,
                           int32_t* kept_per_row, void* hip_stream);

/* Routing baselines for the routing-cost and budget study: the proxy map
 * s_hat = Q_bar K_bar^T / sqrt(d) of every head is materialized, then every
 * row is selected by one of
 *   SOL_ROUTE_THRESHOLD  s_hat_ij > mu_i + beta*sigma_i, mu_i and sigma_i the
 *                        mean and population std of the materialized row
 *                        (page "Sol-Attn: l'attenzione sparsa che sceglie al
 *                        volo" (paithon.it), section "Una soglia per ogni riga");
 *   SOL_ROUTE_TOPK       the row's top_k highest scores, ties to lower j;
 *   SOL_ROUTE_TOPP       the best blocks (ties to lower j) until the softmax
 *                        probability of the row's scores reaches top_p (the
 *                        block that reaches it is kept; all if rounding never
 *                        does); both from the same page, section "Perche
 *                        l'attenzione pesa tanto nei video", which also says
 *                        that both write the full score map and the chosen
 *                        indices to GPU memory before attention starts.
 * The fused pass never builds this map; sol_route exists to measure what it
 * avoids. Needs the pre-pass workspace of the same K (sol_block_summaries);
 * writes qbar into it.
 *   q            device, [B][H][N][d] (bf16, or fp32 with SOL_F32)
 *   proxy_map    device float [B*H*n_b*n_b], written (row-major per head)
 *   mask_bits    device uint64 [B*H*n_b*W], written (layout of sol_debug.mask_bits)
 *   kept_per_row device int32 [B*H*n_b] or NULL
 *   topk_idx     device int32 [B*H*n_b*top_k] or NULL: SOL_ROUTE_TOPK only, the kept
 *                key blocks of each row, best first (only min(top_k, n_b) written)
 * flags: SOL_F32, SOL_SYNC and SOL_LOW_MEMORY (a workspace of that mode's size;
 * routing reads no V^T); SOL_CORRECTION, SOL_CORRECTION_ROW or SOL_DENSE give
 * SOL_ERR_INVALID_ARG. Errors: NaN beta / top_p or negative top_k,
 * unknown mode -> SOL_ERR_INVALID_ARG. The masks feed sol_attn_masked. */
#define SOL_ROUTE_THRESHOLD 0
#define SOL_ROUTE_TOPK      1
#define SOL_ROUTE_TOPP      2
sol_status sol_route(const void* q, int B, int H, int N, int d, unsigned flags, int mode,
                     float beta, int top_k, float top_p, const void* workspace, size_t ws_bytes,
                     float* proxy_map, uint64_t* mask_bits, int32_t* kept_per_row,
                     int32_t* topk_idx, void* hip_stream);

/* Whole forward on a caller stream with a caller workspace:
 * sol_block_summaries followed by sol_attn_fused, i.e. the whole method of
 * page "Sol-Attn: l'attenzione sparsa che sceglie al volo" (paithon.it):
 * block summaries and closed-form thresholds (section "Una soglia per ogni
 * riga"), then the one pass that routes, computes the kept blocks exactly and
 * folds in the others (section "Scegliere mentre si calcola"); the paper
 * abstract names the three parts of that pass. Reentrant: calls with
 * distinct workspaces may run concurrently on different streams. */
sol_status sol_attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int N, int d, float beta, unsigned flags,
                           void* hip_stream, void* workspace, size_t ws_bytes,
                           const sol_debug* dbg);

/* Element strides of one logical [B][H][N][d] tensor whose d values per row
 * are contiguous: element (ib, ih, t, c) is at ib*b + ih*h + t*n + c.
 * Contiguous [B][H][N][d] is {H*N*d, N*d, d}; [B][N][H][d] is {N*H*d, d, H*d};
 * one slice of a packed [B][N][3][H][d] projection is {3*N*H*d, d, 3*H*d}. */
typedef struct sol_strides {
  int64_t b, h, n;
} sol_strides;

/* sol_attn_fwd_ex for tensors in other layouts, so that the kernel drops in
 * where a pipeline keeps its projections (the agihunt.info page on the paper
 * presents the method as a drop-in, training-free replacement of the
 * attention kernel; closing paragraphs). The arithmetic and the result are
 * those of sol_attn_fwd_ex on the same logical tensors, bit for bit.
 *   q_strides, k_strides, v_strides, out_strides: strides of each tensor, or
 *     NULL for contiguous [B][H][N][d]. Every stride of a dimension longer
 *     than 1 must be positive; every stride must be a multiple of 8 elements
 *     (bf16) or 4 (fp32), and n must be below 2^24, else SOL_ERR_INVALID_ARG.
 *     The out rows must not overlap one another or the inputs (not checked
 *     beyond n >= d).
 *   q, k, v, out: 16-byte aligned device pointers (else SOL_ERR_INVALID_ARG).
 * Other arguments, workspace size and errors as sol_attn_fwd_ex. */
sol_status sol_attn_fwd_strided(const void* q, const void* k, const void* v, void* out,
                                int B, int H, int N, int d, const sol_strides* q_strides,
                                const sol_strides* k_strides, const sol_strides* v_strides,
                                const sol_strides* out_strides, float beta, unsigned flags,
                                void* hip_stream, void* workspace, size_t ws_bytes,
                                const sol_debug* dbg);

/* Whole forward on the null stream of the current device with a library-owned
 * workspace (allocated on first use, grown when needed, held until the
 * process ends; calls are serialised by a mutex): the drop-in call of the
 * agihunt.info page on the paper (closing paragraphs: a training-free kernel
 * that replaces attention in an existing pipeline), computing what
 * sol_attn_fwd_ex computes. The null stream does not order work against
 * streams created non-blocking: a caller that produced q, k, v on such a
 * stream must make the null stream wait for it (and its consumers wait for
 * the null stream), or call sol_attn_fwd_ex on that stream. */
sol_status sol_attn_fwd(const void* q, const void* k, const void* v, void* out,
                        int B, int H, int N, int d, float beta, unsigned flags);

/* For callers that cannot allocate device memory: code recorded into a HIP
 * graph, tight serving loops, harnesses that forbid hipMalloc. The same
 * forward as sol_attn_fwd_ex on a caller stream, with no caller workspace: the
 * pre-pass arrays go to a scratch array of 64 MiB in the library's static
 * device memory (one per GPU, held from library load until the process
 * ends), and the call allocates and frees nothing. Shapes whose workspace
 * (sol_attn_workspace_bytes_flags) exceeds 64 MiB give SOL_ERR_UNSUPPORTED before
 * any device work. Every call on one GPU uses that GPU's one scratch array,
 * whose contents the previous call leaves behind (nothing in it has to start
 * at zero): calls that may overlap on one GPU (on different streams, or a
 * replayed graph and another call) race and must be ordered by the caller.
 * Other arguments and errors as sol_attn_fwd_ex. */
sol_status sol_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                                int B, int H, int N, int d, float beta, unsigned flags,
                                void* hip_stream, const sol_debug* dbg);

#ifdef __cplusplus
}
#endif

#endif /* SOL_ATTN_H */
