"""CPU oracle for Sol-Attn's on-the-fly block-sparse attention (forward).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's
cpu_baseline leg may import this module. The HIP library never calls it, and
it shares no code, header, table or helper with the HIP path.

It is the plain, slow, step-by-step statement of what the method computes,
following the pages in their own order and notation:

  page "Sol-Attn: l'attenzione sparsa che sceglie al volo, per generare video
  più in fretta" (paithon.it), cited below as [IT] with its section names;
  page "Sol-Attn: Accelerating Video Generation Inference via On-the-Fly
  Attention Sparsification" (agihunt.info), cited as [EN-agihunt];
  the paper abstract (hotpaper.ai), cited as [abstract].

For each (batch, head) and each 64-token query block i:
  1. block means q_bar_i, k_bar_j, v_bar_j                  [IT, "Perché l'attenzione pesa tanto nei video"]
  2. proxy s_hat_ij = q_bar_i . k_bar_j / sqrt(d)          [IT, same section; the 1/sqrt(d) is our reading]
  3. mu_i, sigma_i = mean and population std of row i      [EN-agihunt, threshold paragraph]
  4. tau_i = mu_i + beta*sigma_i, S_i = {j : s_hat_ij > tau_i}   [IT, "Una soglia per ogni riga", equation]
  5. exact softmax attention over the tokens of the kept blocks, plus, when the
     correction is on, each unselected block entered as 64 virtual tokens whose
     logit is s_hat_ij and whose value is v_bar_j, in the numerator and the
     denominator alike                                     [IT, "Scegliere mentre si calcola", last paragraph]

The oracle computes the whole row of proxy scores and thresholds it offline:
the pages state that the online, in-pass test gives the same result as such
an offline threshold of the full row ([IT], "Scegliere mentre si calcola").

Precision. Attention arithmetic (logits, exponentials, sums, division) is
float64. The routing decision (block means, s_hat, mu, sigma, tau and the
comparison) is taken in `route_dtype`, float32 by default, which is the
precision the GPU kernel takes it in; the pins also run it in float64.
Block means are formed in float64 and then rounded to `route_dtype`.

Readings where the pages are silent (listed with reasons in the design notes):
  * proxy scale 1/sqrt(d); strict '>' ; population std (1/n_b) over all n_b
    key blocks (no causal mask, no forced blocks);
  * beta = -inf keeps every block (tau = -inf, no -inf*0); beta = +inf keeps none;
  * a row with no kept block and the correction off outputs zeros;
  * the correction logit is the block-level s_hat_ij (not a per-row q_r.k_bar_j).

The two routing baselines the pages compare the threshold with, top-k and
top-p, are stated too (select_topk, select_topp); they select from the same
proxy row.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

BLOCK = 64


def block_means(x: np.ndarray) -> np.ndarray:
    """Mean of each 64-token block: [N, d] -> [N/64, d], in float64.

    [IT] "Perché l'attenzione pesa tanto nei video": the sequence is cut into
    64-token blocks and each block is summarised by its mean query / mean key.
    """
    n, d = x.shape
    if n % BLOCK:
        raise ValueError("sequence length must be a multiple of 64")
    return np.asarray(x, dtype=np.float64).reshape(n // BLOCK, BLOCK, d).mean(axis=1)


def proxy_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_hat[i, j] = q_bar_i . k_bar_j / sqrt(d), computed in the dtype of the inputs.

    [IT] "Perché l'attenzione pesa tanto nei video" (product of the block-mean
    query and each block's mean key); the 1/sqrt(d) scale is our reading.
    """
    d = qbar.shape[1]
    scale = qbar.dtype.type(1.0 / math.sqrt(d))
    return (qbar @ kbar.T) * scale


def row_mean_std(s_hat: np.ndarray):
    """Brute-force mean and population standard deviation of each proxy row.

    [EN-agihunt] threshold paragraph: mu_i and sigma_i are the mean and the
    standard deviation of query i's row of proxy scores. Two passes.
    """
    mu = s_hat.mean(axis=1)
    dev = s_hat - mu[:, None]
    sigma = np.sqrt((dev * dev).mean(axis=1))
    return mu, sigma


def key_summary_moments(kbar: np.ndarray):
    """Mean m of the compressed keys and their centred d x d second-moment matrix C.

    [IT] "Una soglia per ogni riga", last paragraph: mu_i and sigma_i follow
    from the mean of the compressed keys and their d x d second-moment matrix.
    C = (1/n_b) sum_j (k_bar_j - m)(k_bar_j - m)^T (population, centred).
    """
    m = kbar.mean(axis=0)
    c = kbar - m[None, :]
    return m, (c.T @ c) / kbar.shape[0]


def closed_form_mean_std(qbar: np.ndarray, m: np.ndarray, C: np.ndarray):
    """mu_i = q_bar_i.m/sqrt(d), sigma_i = sqrt(max(0, q_bar_i^T C q_bar_i)/d).

    The same numbers as row_mean_std of the proxy rows, without forming a row
    ([IT] "Una soglia per ogni riga", last paragraph).
    """
    d = qbar.shape[1]
    mu = (qbar @ m) / math.sqrt(d)
    var = np.einsum("ic,cd,id->i", qbar, C, qbar) / d
    return mu, np.sqrt(np.maximum(var, 0.0))


def thresholds(mu: np.ndarray, sigma: np.ndarray, beta: float) -> np.ndarray:
    """tau_i = mu_i + beta*sigma_i ([IT] "Una soglia per ogni riga", equation).

    beta = -inf gives tau = -inf (every block kept) and beta = +inf gives
    tau = +inf (none kept), without forming beta*sigma when sigma is 0.
    """
    if math.isnan(beta):
        raise ValueError("beta is NaN")
    if beta == -math.inf:
        return np.full_like(mu, -np.inf)
    if beta == math.inf:
        return np.full_like(mu, np.inf)
    return mu + mu.dtype.type(beta) * sigma


def select_blocks(s_hat: np.ndarray, tau: np.ndarray) -> np.ndarray:
    """S_i = {j : s_hat_ij > tau_i}, strict ([IT] "Una soglia per ogni riga", equation)."""
    return s_hat > tau[:, None]


def select_topk(s_hat: np.ndarray, k: int) -> np.ndarray:
    """Top-k routing, the baseline the pages set against the threshold: each row
    keeps its k highest proxy scores ([IT] "Perché l'attenzione pesa tanto nei
    video"). Equal scores are taken in ascending j (reading: the pages give no
    tie rule). k is clamped to [0, n_b]."""
    n_rows, nb = s_hat.shape
    k = max(0, min(int(k), nb))
    keep = np.zeros((n_rows, nb), dtype=bool)
    for i in range(n_rows):
        order = sorted(range(nb), key=lambda j: (-float(s_hat[i, j]), j))
        keep[i, order[:k]] = True
    return keep


def select_topp(s_hat: np.ndarray, p: float) -> np.ndarray:
    """Top-p routing: each row keeps blocks, best proxy score first, until their
    cumulative probability reaches p ([IT] "Perché l'attenzione pesa tanto nei
    video"). Readings: the probability of block j is the softmax of the row's
    proxy scores (the scores as logits); the block whose addition reaches p is
    kept; equal scores are taken in ascending j; when rounding keeps the total
    below p every block is kept. Accumulated in float64."""
    n_rows, nb = s_hat.shape
    keep = np.zeros((n_rows, nb), dtype=bool)
    for i in range(n_rows):
        row = s_hat[i].astype(np.float64)
        w = np.exp(row - row.max())
        prob = w / w.sum()
        order = sorted(range(nb), key=lambda j: (-float(s_hat[i, j]), j))
        acc = 0.0
        for j in order:
            keep[i, j] = True
            acc += prob[j]
            if acc >= p:
                break
    return keep


def _attend_query_block(qi: np.ndarray, k: np.ndarray, v: np.ndarray, keep: np.ndarray,
                        s_hat_row: np.ndarray, vbar: np.ndarray, correction: bool,
                        kbar_rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Output rows of one query block: exact tokens of kept blocks + virtual tokens.

    [IT] "Scegliere mentre si calcola", last paragraph: every token of an
    excluded block is treated as carrying the block-mean key, and its term
    enters both the numerator and the denominator of the softmax; the logit
    reused is the block's proxy score. Form: 64 virtual tokens with logit
    s_hat_ij and value v_bar_j per unselected block j.

    With kbar_rows (the float64 block-mean keys) the virtual tokens of row r
    take the per-row logit q_r . k_bar_j / sqrt(d) instead: the literal reading
    of "each token takes the block-mean key" (exact when a block's 64 keys are
    equal), which the pages leave beside the block-level reuse.
    """
    d = qi.shape[1]
    kept = np.flatnonzero(keep)
    dropped = np.flatnonzero(~keep)
    kb = k.reshape(-1, BLOCK, d)
    vb = v.reshape(-1, BLOCK, d)
    k_kept = kb[kept].reshape(-1, d)
    v_kept = vb[kept].reshape(-1, d)

    logits = (qi @ k_kept.T) / math.sqrt(d)                 # [64, 64*|S_i|]
    rows = qi.shape[0]
    if correction and dropped.size:
        if kbar_rows is None:                                 # block-level logit, same for every row
            virt = np.broadcast_to(np.asarray(s_hat_row[dropped], dtype=np.float64)[None, :],
                                   (rows, dropped.size))
        else:                                                 # per-row logit
            virt = (qi @ kbar_rows[dropped].T) / math.sqrt(d)
    else:
        virt = np.zeros((rows, 0), dtype=np.float64)

    out = np.zeros((rows, d), dtype=np.float64)
    if logits.shape[1] == 0 and virt.shape[1] == 0:
        return out                                             # nothing to attend to
    row_max = np.full(rows, -np.inf)
    if logits.shape[1]:
        row_max = logits.max(axis=1)
    if virt.shape[1]:
        row_max = np.maximum(row_max, virt.max(axis=1))
    num = np.zeros((rows, d))
    den = np.zeros(rows)
    if logits.shape[1]:
        p = np.exp(logits - row_max[:, None])
        num += p @ v_kept
        den += p.sum(axis=1)
    if virt.shape[1]:
        w = BLOCK * np.exp(virt - row_max[:, None])            # [64, n_drop]
        num += w @ vbar[dropped]
        den += w.sum(axis=1)
    return num / den[:, None]


def sol_attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, beta: float,
                       correction: bool = True, *,
                       query_blocks: Optional[Sequence[int]] = None,
                       mask_override: Optional[np.ndarray] = None,
                       route_dtype=np.float32,
                       correction_form: str = "block",
                       text_blocks: int = 0) -> Dict[str, np.ndarray]:
    """Sol-Attn forward for one head. q, k, v: [N, d] (any float dtype; upcast to float64).

    Returns a dict with
      out    [len(query_blocks)*64, d] float64 (rows of the requested query blocks, in order)
      mask   [len(query_blocks), n_b] bool, the kept set S_i used
      s_hat, mu, sigma, tau   routing quantities of the requested rows (route_dtype)
      kept   [len(query_blocks)] int, |S_i|
    mask_override, if given ([len(query_blocks), n_b] bool), replaces S_i for the
    attention step (routing quantities are still returned), so that arithmetic
    can be compared separately from the selection.
    correction_form: "block" (the logit of a block's virtual tokens is s_hat_ij)
    or "row" (q_r . k_bar_j / sqrt(d) for row r, see _attend_query_block).
    text_blocks: joint attention with a text segment of that many blocks at the
    end of the sequence, always computed exactly ([IT] "Dove leggere con
    attenzione": text tokens in joint attention are always exact). Reading: the
    selection runs as usual over all n_b key blocks, then every query block
    keeps the text key blocks and a text query block keeps every key block.
    """
    if correction_form not in ("block", "row"):
        raise ValueError("correction_form must be 'block' or 'row'")
    q64 = np.asarray(q, dtype=np.float64)
    k64 = np.asarray(k, dtype=np.float64)
    v64 = np.asarray(v, dtype=np.float64)
    n, d = q64.shape
    nb = n // BLOCK
    qb = np.arange(nb) if query_blocks is None else np.asarray(query_blocks, dtype=np.int64)

    kbar = block_means(k64).astype(route_dtype)
    qbar = block_means(q64)[qb].astype(route_dtype)
    vbar = block_means(v64)
    s_hat = proxy_scores(qbar, kbar)
    mu, sigma = row_mean_std(s_hat)
    tau = thresholds(mu, sigma, beta)
    mask = select_blocks(s_hat, tau)
    if text_blocks:
        t0 = nb - int(text_blocks)
        mask[:, t0:] = True
        mask[qb >= t0, :] = True
    use = mask if mask_override is None else np.asarray(mask_override, dtype=bool)

    kbar_rows = block_means(k64) if correction_form == "row" else None
    out = np.empty((qb.size * BLOCK, d), dtype=np.float64)
    for r, i in enumerate(qb):
        qi = q64[i * BLOCK:(i + 1) * BLOCK]
        out[r * BLOCK:(r + 1) * BLOCK] = _attend_query_block(
            qi, k64, v64, use[r], s_hat[r], vbar, correction,
            kbar_rows=kbar_rows)
    return {"out": out, "mask": mask, "s_hat": s_hat, "mu": mu, "sigma": sigma,
            "tau": tau, "kept": mask.sum(axis=1)}


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Textbook softmax attention softmax(q k^T / sqrt(d)) v for one head, float64.

    Written separately from the sparse path (it is the dense baseline the
    method replaces, [EN-agihunt] drop-in statement).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    z = (q @ k.T) / math.sqrt(q.shape[1])
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e @ v) / e.sum(axis=1, keepdims=True)
