"""Plain float64 reference for block-sparse landmark attention (numpy only).

TEST INFRASTRUCTURE ONLY -- imported by the tests, the smoke check and the benchmark's
CPU-baseline leg, never by the product path.  Page titles are listed in oracle/__init__.py.

What is computed, step by step, in the pages' order:

1. landmarks   -- neighbouring keys pooled into one vector per block (LSA page, "The index
                  stops scanning the whole context", paragraph 3: neighbouring keys are merged
                  first to make indexing cheaper; the HiLS page names such per-chunk vectors
                  "landmarks").  The pooling is the mean over a block of 64 tokens, stored in
                  the input dtype (round-to-nearest-even).
2. selector    -- one query vector per (kv group, query block): the mean of the block's queries,
                  summed over the query heads that share the kv head.  Kept in float64.
3. scores      -- selector . landmark for every block up to the current one (SAS page, summary
                  paragraph 1: a light selector scores the units of context; LSA page, first
                  section, paragraph 2: the indexer scores each contiguous block).
4. selection   -- hard top-K over the scores (SAS page, summary paragraph 1, and "How to apply":
                  hard top-K is what inference uses), plus the start of the context and a recent
                  window that are always attended (LSA page, first section, paragraph 4), the
                  current block always kept (SAS page, summary paragraph 3).  Ties: lower block
                  index wins.
5. SAS gate    -- a continuous selector score turned into a log-form gate that sits inside the
                  softmax and is normalised against the always-kept current block (SAS page,
                  summary paragraph 3 and "Key facts" item 3): g_j = log sigmoid(S_j - S_c).
6. attention   -- softmax over the attended keys (blocks of A_c, causal inside the current
                  block), with the gate added to every logit of its block.
7. HiLS        -- each query attends to each selected chunk on its own, then the chunk outputs
                  are merged with weights equal to the chunks' retrieval scores (HiLS page,
                  summary paragraph 2); the retrieval score is softmax_j(q . L_j / sqrt(D)).
8. paged decode -- the decode step of a ragged batch whose cache lives in 64-token pages: each
                  sequence is the contiguous decode step of its own tokens, read through its
                  page table (the serving layout; the pages say nothing of storage, so the
                  method is unchanged by it).
9. backward    -- gradients of the attention step for given attended sets: into q, k, v; for
                  SAS into the selector scores through the gates (the pages train the selector
                  end to end through these gates); for HiLS into the landmarks through the
                  retrieval scores.
10. LSA index   -- the flat clustered indexer: Ward clusters of the landmarks of each completed
                  segment, kept as centres plus member tables; a query scores the centres and
                  the best clusters are expanded back to blocks (LSA page, "The index stops
                  scanning the whole context", paragraphs 3-5).
11. LSA tree    -- the same clusters under segments and groups of segments, walked by beam
                  search (the same page, paragraph 5).

Readings taken where the pages are silent (each is listed in the design notes):
* the selector vector is kept in float64 here (float32 on the device), never rounded to bf16;
* the selector score carries no 1/sqrt(D) (ranking does not depend on it);
* K counts the extra blocks beyond the sink and the local window: candidates are the blocks
  j with n_sink <= j <= c - n_local;
* the SAS gate is added after the logits are scaled by 1/sqrt(D); the current block's gate
  is 0; every other attended block (sink, local, top-K) is gated;
* HiLS retrieval scores use each token's own query of its own head, scaled by 1/sqrt(D),
  softmax-normalised over all attended chunks, with the current chunk's full-block landmark;
* a partial last block (T not a multiple of 64) pools over the tokens present;
* paged decode: a page holds one 64-token block of every kv head, [n_pages, Hkv, 64, D].
"""

from __future__ import annotations

import math

import numpy as np

BLOCK = 64


# --------------------------------------------------------------------------------------
# rounding to the input dtype
# --------------------------------------------------------------------------------------

def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of `dtype` ("f32" or "bf16"), ties to even.

    The result is returned as float64 holding exactly representable values of `dtype`.
    bf16 keeps 8 significant bits (1 implicit + 7 stored) with float32's exponent range.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(f"unknown dtype {dtype!r}")
    out = np.empty_like(x)
    finite = np.isfinite(x)
    xf = x[finite]
    mant, expo = np.frexp(xf)                     # xf = mant * 2**expo, 0.5 <= |mant| < 1
    # below the smallest normal (2**-126) the quantum is fixed at 2**-133
    expo = np.maximum(expo, -125)
    q = np.ldexp(np.rint(np.ldexp(xf, 8 - expo)), expo - 8)   # np.rint rounds half to even
    q = np.where(np.abs(q) > 3.3895313892515355e38, np.copysign(np.inf, xf), q)
    out[finite] = q
    out[~finite] = x[~finite]
    return out


# --------------------------------------------------------------------------------------
# 1. landmarks
# --------------------------------------------------------------------------------------

def n_blocks(T: int, block: int = BLOCK) -> int:
    return (T + block - 1) // block


def landmarks(k: np.ndarray, dtype: str, block: int = BLOCK) -> np.ndarray:
    """L[b,h,j,:] = mean of k[b,h,t,:] over the tokens t of block j, rounded to `dtype`.

    LSA page, "The index stops scanning the whole context", paragraph 3 (neighbouring keys
    are pooled before indexing); the pooling is the block mean.  k: [B,H,T,D] float64.
    """
    B, H, T, D = k.shape
    NB = n_blocks(T, block)
    L = np.empty((B, H, NB, D), dtype=np.float64)
    for j in range(NB):
        lo, hi = j * block, min((j + 1) * block, T)
        L[:, :, j, :] = k[:, :, lo:hi, :].mean(axis=2)
    return round_to_dtype(L, dtype)


# --------------------------------------------------------------------------------------
# 2. selector vectors
# --------------------------------------------------------------------------------------

def selector_vectors(q: np.ndarray, n_kv_heads: int, block: int = BLOCK) -> np.ndarray:
    """qbar[b,g,c,:] = sum over the query heads h of kv group g of mean_{t in block c} q[b,h,t,:].

    Query head h belongs to kv group h // (Hq / Hkv).  q: [B,Hq,T,D] float64.  Float64 result,
    not rounded.
    """
    B, Hq, T, D = q.shape
    G = Hq // n_kv_heads
    NQB = n_blocks(T, block)
    qbar = np.zeros((B, n_kv_heads, NQB, D), dtype=np.float64)
    for c in range(NQB):
        lo, hi = c * block, min((c + 1) * block, T)
        m = q[:, :, lo:hi, :].mean(axis=2)              # [B,Hq,D]
        qbar[:, :, c, :] = m.reshape(B, n_kv_heads, G, D).sum(axis=2)
    return qbar


def decode_selector_vectors(q: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """Decode: the one query token per sequence, summed over the heads of each kv group.

    q: [B,Hq,D] -> [B,Hkv,D] float64.
    """
    B, Hq, D = q.shape
    G = Hq // n_kv_heads
    return q.reshape(B, n_kv_heads, G, D).sum(axis=2)


# --------------------------------------------------------------------------------------
# 3. scores
# --------------------------------------------------------------------------------------

def block_scores(qbar: np.ndarray, L: np.ndarray) -> np.ndarray:
    """S[..., c, j] = qbar[..., c, :] . L[..., j, :] in float64 (a plain matrix product).

    SAS page, summary paragraph 1 (a light selector scores each unit of context); LSA page,
    first section, paragraph 2 (each contiguous block is scored).  Entries with j > c are
    computed too but are never read.
    """
    return np.matmul(qbar, np.swapaxes(L, -1, -2))


# --------------------------------------------------------------------------------------
# 4. selection
# --------------------------------------------------------------------------------------

def select_row(s_row: np.ndarray, c: int, topk: int, n_sink: int = 1, n_local: int = 2):
    """Attended block set A_c of query block c, ascending, and the scores aligned with it.

    * hard top-K over the selector scores (SAS page, summary paragraph 1; "How to apply");
    * the start of the context (n_sink blocks) and a recent window (n_local blocks ending
      at the current one) are always attended (LSA page, first section, paragraph 4);
    * the current block c is always kept (SAS page, summary paragraph 3).
    Candidates are the blocks j with n_sink <= j <= c - n_local; they are ranked by score,
    descending, and among equal scores the lower block index ranks first.
    """
    s_row = np.asarray(s_row, dtype=np.float64)
    sink = set(range(0, min(n_sink, c + 1)))
    local = set(range(max(0, c - n_local + 1), c + 1))
    cand = np.arange(n_sink, c - n_local + 1, dtype=np.int64)
    if cand.size:
        # np.lexsort sorts by the last key first: primary -score (descending), then index
        order = np.lexsort((cand, -s_row[cand]))
        top = set(cand[order[: min(topk, cand.size)]].tolist())
    else:
        top = set()
    A = np.array(sorted(sink | local | top), dtype=np.int64)
    return A, s_row[A]


def select_all(S: np.ndarray, topk: int, n_sink: int = 1, n_local: int = 2, row_blocks=None):
    """Selection for every row of S[B,G,R,NB].

    row_blocks[r] is the query block index c of row r (prefill: r itself; decode: the block of
    the last token).  Returns idx [B,G,R,NA] int64 padded with -1 and sc [B,G,R,NA] float64
    (NaN in the padding), NA = n_sink + n_local + topk.
    """
    B, G, R, NB = S.shape
    NA = n_sink + n_local + topk
    if row_blocks is None:
        row_blocks = list(range(R))
    idx = np.full((B, G, R, NA), -1, dtype=np.int64)
    sc = np.full((B, G, R, NA), np.nan, dtype=np.float64)
    for b in range(B):
        for g in range(G):
            for r in range(R):
                A, sA = select_row(S[b, g, r], row_blocks[r], topk, n_sink, n_local)
                idx[b, g, r, : A.size] = A
                sc[b, g, r, : A.size] = sA
    return idx, sc


# --------------------------------------------------------------------------------------
# 5. SAS gate
# --------------------------------------------------------------------------------------

def log_sigmoid(x) -> np.ndarray:
    """log(1 / (1 + exp(-x))), evaluated without overflow on either side."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-np.abs(x))), x - np.log1p(np.exp(-np.abs(x))))


def sas_gates(A: np.ndarray, sA: np.ndarray, c: int) -> np.ndarray:
    """Gate per attended block: log sigmoid(S_j - S_c) for j != c, 0 for the current block.

    SAS page, summary paragraph 3 and "Key facts" item 3: the continuous selector score enters
    the softmax in log form, normalised so that earlier context is compared with the current
    block, which is always kept.
    """
    A = np.asarray(A)
    sA = np.asarray(sA, dtype=np.float64)
    s_c = sA[np.nonzero(A == c)[0][0]]
    g = log_sigmoid(sA - s_c)
    g[A == c] = 0.0
    return g


# --------------------------------------------------------------------------------------
# 6. attention (PLAIN / SAS)
# --------------------------------------------------------------------------------------

def _block_keys(A, T: int, block: int):
    """Key positions of the attended blocks (ascending) and the block of each position."""
    pos, blk = [], []
    for j in A:
        lo, hi = int(j) * block, min((int(j) + 1) * block, T)
        pos.extend(range(lo, hi))
        blk.extend([int(j)] * (hi - lo))
    return np.array(pos, dtype=np.int64), np.array(blk, dtype=np.int64)


def attend_rows(qrows, tpos, K, V, A, gates, scale: float, block: int = BLOCK):
    """Softmax attention of query rows over the keys of the attended blocks.

    qrows [m,D] (rows of one head), tpos [m] their token positions, K/V [T,D] that head's kv
    group, A the attended blocks, gates aligned with A (zeros for PLAIN).  For row t the
    visible keys are u in the blocks of A with u <= t; logit = scale * q.k_u + gate(block(u)).
    Returns out [m,D] and lse [m] = log sum_u exp(logit_u).
    """
    T = K.shape[0]
    pos, blk = _block_keys(A, T, block)
    gate_of = dict(zip([int(a) for a in A], np.asarray(gates, dtype=np.float64)))
    gvec = np.array([gate_of[int(j)] for j in blk], dtype=np.float64)
    logits = scale * (qrows @ K[pos].T) + gvec[None, :]            # [m, |U|]
    visible = pos[None, :] <= np.asarray(tpos)[:, None]
    logits = np.where(visible, logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    den = e.sum(axis=1, keepdims=True)
    out = (e / den) @ V[pos]
    lse = (mx + np.log(den))[:, 0]
    return out, lse


# --------------------------------------------------------------------------------------
# 7. HiLS
# --------------------------------------------------------------------------------------

def hils_chunks(qrows, tpos, K, V, A, scale: float, block: int = BLOCK):
    """Per-chunk attention: each query attends to each attended chunk on its own.

    HiLS page, summary paragraph 2 (each query first looks at each selected chunk
    independently).  Returns o_j [m,|A|,D] (softmax over the visible keys of chunk j only) and
    lse_j [m,|A|].  Every chunk in A holds at least one visible key for every row, because the
    current chunk contains the row's own position.
    """
    m = qrows.shape[0]
    o = np.zeros((m, len(A), V.shape[1]))
    lse = np.zeros((m, len(A)))
    for i, j in enumerate(A):
        o[:, i, :], lse[:, i] = attend_rows(qrows, tpos, K, V, [j], [0.0], scale, block)
    return o, lse


def attend_hils_rows(qrows, tpos, K, V, Lrows, A, scale: float, block: int = BLOCK):
    """HiLS output: o = sum_j w_j o_j with w = softmax_j(scale * q . L_j) over attended chunks.

    HiLS page, summary paragraph 2: the chunk results are combined with weights equal to the
    chunks' retrieval scores.  Lrows [|A|,D] are the landmarks of the chunks in A.
    """
    o_j, _ = hils_chunks(qrows, tpos, K, V, A, scale, block)
    r = scale * (qrows @ Lrows.T)                                    # [m, |A|]
    w = np.exp(r - r.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)
    return np.einsum("ma,mad->md", w, o_j)


# --------------------------------------------------------------------------------------
# whole path
# --------------------------------------------------------------------------------------

def _default_scale(D, scale):
    return 1.0 / math.sqrt(D) if not scale else float(scale)


def prefill_rows(q, k, v, rows, *, topk: int, mode: str, dtype: str, block: int = BLOCK,
                 n_sink: int = 1, n_local: int = 2, scale=None, idx=None, lm=None, qbar=None):
    """Prefill outputs for a subset of (b, g, c) rows: all query heads of group g, block c.

    q [B,Hq,T,D], k/v [B,Hkv,T,D] float64 holding the exact input values.  `rows` is a list of
    (b, g, c).  If `idx` [B,Hkv,NQB,NA] is given, those attended sets are used instead of the
    oracle's own selection (scores and gates still come from the oracle's own landmarks and
    selector vectors).  Returns a dict of per-row results keyed by (b, g, c):
    {"A", "sA", "out" [G,nrows,D], "lse" [G,nrows] (PLAIN/SAS)}.
    """
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc_ = _default_scale(D, scale)
    if lm is None:
        lm = landmarks(k, dtype, block)
    if qbar is None:
        qbar = selector_vectors(q, Hkv, block)
    res = {}
    for (b, g, c) in rows:
        s_row = block_scores(qbar[b, g, c][None, :], lm[b, g])[0]     # [NB]
        if idx is None:
            A, sA = select_row(s_row, c, topk, n_sink, n_local)
        else:
            A = np.array([j for j in idx[b, g, c] if j >= 0], dtype=np.int64)
            sA = s_row[A]
        lo, hi = c * block, min((c + 1) * block, T)
        tpos = np.arange(lo, hi)
        outs, lses = [], []
        for hh in range(G):
            h = g * G + hh
            qr = q[b, h, lo:hi]
            if mode == "hils":
                o = attend_hils_rows(qr, tpos, k[b, g], v[b, g], lm[b, g][A], A, sc_, block)
                lse = np.full(hi - lo, np.nan)
            else:
                gates = sas_gates(A, sA, c) if mode == "sas" else np.zeros(len(A))
                o, lse = attend_rows(qr, tpos, k[b, g], v[b, g], A, gates, sc_, block)
            outs.append(o)
            lses.append(lse)
        res[(b, g, c)] = {"A": A, "sA": sA, "out": np.stack(outs), "lse": np.stack(lses)}
    return res


def prefill(q, k, v, *, topk: int, mode: str, dtype: str, block: int = BLOCK, n_sink: int = 1,
            n_local: int = 2, scale=None, idx=None):
    """Whole prefill pass: landmarks, selector vectors, scores, selection and attention.

    Returns a dict with lm [B,Hkv,NB,D], qbar [B,Hkv,NQB,D], S [B,Hkv,NQB,NB], idx/sc
    [B,Hkv,NQB,NA], out [B,Hq,T,D] and lse [B,Hq,T] (NaN for HiLS).
    """
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    NQB = n_blocks(T, block)
    lm = landmarks(k, dtype, block)
    qbar = selector_vectors(q, Hkv, block)
    S = block_scores(qbar, lm)
    own_idx, own_sc = select_all(S, topk, n_sink, n_local)
    rows = [(b, g, c) for b in range(B) for g in range(Hkv) for c in range(NQB)]
    per = prefill_rows(q, k, v, rows, topk=topk, mode=mode, dtype=dtype, block=block,
                       n_sink=n_sink, n_local=n_local, scale=scale, idx=idx, lm=lm, qbar=qbar)
    out = np.zeros((B, Hq, T, D))
    lse = np.zeros((B, Hq, T))
    for (b, g, c), r in per.items():
        lo, hi = c * block, min((c + 1) * block, T)
        out[b, g * G:(g + 1) * G, lo:hi] = r["out"]
        lse[b, g * G:(g + 1) * G, lo:hi] = r["lse"]
    return {"lm": lm, "qbar": qbar, "S": S, "idx": own_idx, "sc": own_sc, "out": out, "lse": lse}


def decode(q, kc, vc, lm, *, topk: int, mode: str, block: int = BLOCK, n_sink: int = 1,
           n_local: int = 2, scale=None, idx=None, seqs=None, groups=None):
    """Decode step: the query is the last cached token (position Tk - 1) of each sequence.

    q [B,Hq,D]; kc/vc [B,Hkv,Tk,D] (the cache includes the query's own key and value);
    lm [B,Hkv,NB,D] the pooled cache.  Selection uses the heads of each kv group summed;
    attention covers every key of the attended blocks (all are at or before Tk - 1).
    Optional `seqs`/`groups` restrict the (b, g) pairs computed.  Returns a dict with
    idx/sc [B,Hkv,NA] (for the computed pairs), out [B,Hq,D] and lse [B,Hq].
    """
    B, Hq, D = q.shape
    Hkv, Tk = kc.shape[1], kc.shape[2]
    G = Hq // Hkv
    sc_ = _default_scale(D, scale)
    c = (Tk - 1) // block
    qbar = decode_selector_vectors(q, Hkv)
    NA = n_sink + n_local + topk
    out_idx = np.full((B, Hkv, NA), -1, dtype=np.int64)
    out_sc = np.full((B, Hkv, NA), np.nan)
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        for g in (range(Hkv) if groups is None else groups):
            s_row = block_scores(qbar[b, g][None, :], lm[b, g])[0]
            if idx is None:
                A, sA = select_row(s_row, c, topk, n_sink, n_local)
            else:
                A = np.array([j for j in idx[b, g] if j >= 0], dtype=np.int64)
                sA = s_row[A]
            out_idx[b, g, : A.size] = A
            out_sc[b, g, : A.size] = sA
            for hh in range(G):
                h = g * G + hh
                qr = q[b, h][None, :]
                tpos = np.array([Tk - 1])
                if mode == "hils":
                    o = attend_hils_rows(qr, tpos, kc[b, g], vc[b, g], lm[b, g][A], A, sc_, block)
                    out[b, h] = o[0]
                else:
                    gates = sas_gates(A, sA, c) if mode == "sas" else np.zeros(len(A))
                    o, l_ = attend_rows(qr, tpos, kc[b, g], vc[b, g], A, gates, sc_, block)
                    out[b, h], lse[b, h] = o[0], l_[0]
    return {"idx": out_idx, "sc": out_sc, "out": out, "lse": lse, "qbar": qbar}


# ---------------------------------------------------------------------------------------------
# paged, ragged decode (the serving layout of the decode step)
# ---------------------------------------------------------------------------------------------
# Readings: a page holds one 64-token block of every kv head, pool [n_pages, Hkv, 64, D]; block j
# of sequence b is page page_table[b, j]; sequence b holds seq_lens[b] tokens.  The method is
# unchanged by the storage: each sequence is the contiguous decode step of its own first
# seq_lens[b] tokens (LSA page, first section, paragraph 4 and "The index stops scanning the
# whole context", paragraph 3: the cache is pooled and scanned per sequence; the pages only say
# where its blocks live).

def gather_pages(pool: np.ndarray, table_row, n_tokens: int, block: int = BLOCK) -> np.ndarray:
    """The first n_tokens of one sequence's cache read through its page table: [Hkv, n_tokens, D]."""
    tiles = [pool[int(table_row[j])] for j in range(n_blocks(n_tokens, block))]
    return np.concatenate(tiles, axis=1)[:, :n_tokens]


def decode_paged(q, k_pool, v_pool, page_table, seq_lens, *, topk: int, mode: str, dtype: str,
                 block: int = BLOCK, n_sink: int = 1, n_local: int = 2, scale=None):
    """Paged decode step: sequence b is `decode` on its gathered cache of seq_lens[b] tokens.

    q [B,Hq,D]; k_pool/v_pool [n_pages,Hkv,64,D]; page_table [B,NB]; seq_lens [B].
    Returns out [B,Hq,D], lse [B,Hq], idx/sc [B,Hkv,NA] and lm [B,Hkv,NB,D] (the landmarks of
    each sequence's blocks, zeros past its end).
    """
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    NB = page_table.shape[1]
    NA = n_sink + n_local + topk
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    idx = np.full((B, Hkv, NA), -1, dtype=np.int64)
    sc = np.full((B, Hkv, NA), np.nan)
    lm = np.zeros((B, Hkv, NB, D))
    for b in range(B):
        n = int(seq_lens[b])
        kc = gather_pages(k_pool, page_table[b], n, block)[None]
        vc = gather_pages(v_pool, page_table[b], n, block)[None]
        lm_b = landmarks(kc, dtype, block)
        r = decode(q[b:b + 1], kc, vc, lm_b, topk=topk, mode=mode, block=block, n_sink=n_sink,
                   n_local=n_local, scale=scale)
        out[b], lse[b], idx[b], sc[b] = r["out"][0], r["lse"][0], r["idx"][0], r["sc"][0]
        lm[b, :, : lm_b.shape[2]] = lm_b[0]
    return {"out": out, "lse": lse, "idx": idx, "sc": sc, "lm": lm}


# ---------------------------------------------------------------------------------------------
# backward pass of PLAIN / SAS prefill attention
# ---------------------------------------------------------------------------------------------
# The gradients of the attention step (steps 5-6) with respect to q, k, v and to the selector
# scores that feed the SAS gates, for given attended sets: the pages train the selector end to
# end through these gates (SAS page, summary paragraphs 2-3: the continuous score enters the
# softmax as a log gate so the selector is trained by the task loss).  Standard softmax calculus,
# written out per query row:
#   x_u = scale q.k_u + g_{j(u)},  P_u = exp(x_u - lse),  o = sum_u P_u v_u
#   dv_u += P_u do,  dP_u = do.v_u,  dx_u = P_u (dP_u - do.o),
#   dq = scale sum_u dx_u k_u,  dk_u += scale dx_u q,  dg_j += sum_{u in block j} dx_u,
#   g_j = log sigmoid(S_j - S_c):  dS_j += dg_j sigmoid(S_c - S_j),  dS_c -= the same  (j != c).

def attend_rows_grad(qrows, tpos, K, V, A, gates, scale: float, dout, block: int = BLOCK):
    """Gradients of attend_rows for one head's rows.

    Returns dq [m,D], pos (the attended key positions, ascending, each once), dK and dV [|pos|,D]
    (the gradients of the keys and values at pos) and dgates aligned with A (the summed logit
    gradient of each attended block).
    """
    T = K.shape[0]
    pos, blk = _block_keys(A, T, block)
    gate_of = dict(zip([int(a) for a in A], np.asarray(gates, dtype=np.float64)))
    gvec = np.array([gate_of[int(j)] for j in blk], dtype=np.float64)
    logits = scale * (qrows @ K[pos].T) + gvec[None, :]
    visible = pos[None, :] <= np.asarray(tpos)[:, None]
    logits = np.where(visible, logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    P = e / e.sum(axis=1, keepdims=True)                              # [m, |U|]
    out = P @ V[pos]
    dP = dout @ V[pos].T                                              # [m, |U|]
    dx = P * (dP - np.sum(dout * out, axis=1, keepdims=True))
    dq = scale * (dx @ K[pos])
    dK = scale * (dx.T @ qrows)
    dV = P.T @ dout
    col = dx.sum(axis=0)
    dg = np.array([col[blk == int(j)].sum() for j in A])
    return dq, pos, dK, dV, dg


def sas_gates_grad(A, sA, c: int, dg) -> np.ndarray:
    """Gradient with respect to the scores sA listed beside A, given dg = d loss / d gate."""
    A = np.asarray(A)
    sA = np.asarray(sA, dtype=np.float64)
    d = np.zeros(len(A))
    ic = int(np.nonzero(A == c)[0][0])
    for i, j in enumerate(A):
        if int(j) == c:
            continue
        w = dg[i] / (1.0 + np.exp(sA[i] - sA[ic]))        # dg * sigmoid(S_c - S_j)
        d[i] += w
        d[ic] -= w
    return d


def hils_rows_grad(qrows, tpos, K, V, Lrows, A, scale: float, dout, block: int = BLOCK):
    """Gradients of attend_hils_rows for one head's rows.

    With o_j the softmax attention of a row over the visible keys of chunk j alone,
    w = softmax_j(scale * q . L_j) and o = sum_j w_j o_j (HiLS page, summary paragraph 2):
      dw_j = dout . o_j,  dr_j = w_j (dw_j - sum_i w_i dw_i)  (softmax backward),
      each chunk is a softmax attention with output gradient w_j dout,
      dq = sum over chunks of the attention gradient + scale * sum_j dr_j L_j,
      dL_j = scale * sum_rows dr_j q.
    Returns dq [m,D], pos (attended key positions, ascending, each once), dK, dV [|pos|,D] and
    dL [|A|,D] aligned with A.
    """
    T, D = K.shape
    m = qrows.shape[0]
    tpos = np.asarray(tpos)
    r = scale * (qrows @ Lrows.T)
    w = np.exp(r - r.max(axis=1, keepdims=True))
    w = w / w.sum(axis=1, keepdims=True)                               # [m, |A|]
    pos, blk = _block_keys(A, T, block)
    dq = np.zeros((m, D))
    dK = np.zeros((pos.size, D))
    dV = np.zeros((pos.size, D))
    dw = np.zeros((m, len(A)))
    chunks = []
    for i, j in enumerate(A):
        sel = np.nonzero(blk == int(j))[0]
        keys = pos[sel]
        logits = scale * (qrows @ K[keys].T)
        logits = np.where(keys[None, :] <= tpos[:, None], logits, -np.inf)
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        P = e / e.sum(axis=1, keepdims=True)
        o_j = P @ V[keys]
        dw[:, i] = np.sum(dout * o_j, axis=1)
        chunks.append((sel, keys, P, o_j))
    dr = w * (dw - np.sum(w * dw, axis=1, keepdims=True))
    dq += scale * (dr @ Lrows)
    dL = scale * (dr.T @ qrows)
    for i, (sel, keys, P, o_j) in enumerate(chunks):
        dOj = w[:, i:i + 1] * dout
        dP = dOj @ V[keys].T
        dx = P * (dP - np.sum(dOj * o_j, axis=1, keepdims=True))
        dq += scale * (dx @ K[keys])
        dK[sel] += scale * (dx.T @ qrows)
        dV[sel] += P.T @ dOj
    return dq, pos, dK, dV, dL


def prefill_backward(q, k, v, idx, sc, dout, *, mode: str, block: int = BLOCK, scale=None,
                     lm=None):
    """Backward of prefill attention for the attended sets idx [B,Hkv,NQB,NA]: for SAS the
    scores sc aligned with them form the gates; for HiLS lm [B,Hkv,NB,D] are the landmarks the
    forward used (its retrieval scores).

    Returns dq [B,Hq,T,D], dk, dv [B,Hkv,T,D], dsc [B,Hkv,NQB,NA] (zero for PLAIN and HiLS and
    in the padding) and, for HiLS, dlm [B,Hkv,NB,D] (the gradient of the landmark values; dk
    does not include the pooling that produced them).
    """
    if mode == "hils":
        return _hils_backward(q, k, v, idx, lm, dout, block=block, scale=scale)
    if mode not in ("plain", "sas"):
        raise ValueError("mode must be plain, sas or hils")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc_ = _default_scale(D, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsc = np.zeros(idx.shape)
    for b in range(B):
        for g in range(Hkv):
            for c in range(idx.shape[2]):
                valid = [i for i, j in enumerate(idx[b, g, c]) if j >= 0]
                if not valid:
                    continue
                A = np.array([idx[b, g, c, i] for i in valid], dtype=np.int64)
                sA = np.array([sc[b, g, c, i] for i in valid], dtype=np.float64)
                gates = sas_gates(A, sA, c) if mode == "sas" else np.zeros(len(A))
                lo, hi = c * block, min((c + 1) * block, T)
                tpos = np.arange(lo, hi)
                dg = np.zeros(len(A))
                for hh in range(G):
                    h = g * G + hh
                    dq_h, pos, dK, dV, dg_h = attend_rows_grad(q[b, h, lo:hi], tpos, k[b, g],
                                                               v[b, g], A, gates, sc_,
                                                               dout[b, h, lo:hi], block)
                    dq[b, h, lo:hi] += dq_h
                    dk[b, g, pos] += dK          # pos holds each key once
                    dv[b, g, pos] += dV
                    dg += dg_h
                if mode == "sas":
                    dsc[b, g, c, valid] = sas_gates_grad(A, sA, c, dg)
    return {"dq": dq, "dk": dk, "dv": dv, "dsc": dsc}


def _hils_backward(q, k, v, idx, lm, dout, *, block: int = BLOCK, scale=None):
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc_ = _default_scale(D, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlm = np.zeros(lm.shape)
    for b in range(B):
        for g in range(Hkv):
            for c in range(idx.shape[2]):
                A = np.array([int(j) for j in idx[b, g, c] if j >= 0], dtype=np.int64)
                if A.size == 0:
                    continue
                lo, hi = c * block, min((c + 1) * block, T)
                tpos = np.arange(lo, hi)
                for hh in range(G):
                    h = g * G + hh
                    dq_h, pos, dK, dV, dL = hils_rows_grad(q[b, h, lo:hi], tpos, k[b, g], v[b, g],
                                                          lm[b, g, A], A, sc_, dout[b, h, lo:hi],
                                                          block)
                    dq[b, h, lo:hi] += dq_h
                    dk[b, g, pos] += dK
                    dv[b, g, pos] += dV
                    dlm[b, g, A] += dL
    return {"dq": dq, "dk": dk, "dv": dv, "dsc": np.zeros(idx.shape), "dlm": dlm}


# --------------------------------------------------------------------------------------
# 10. LSA flat clustered index (Ward clustering of the landmarks of completed segments)
# --------------------------------------------------------------------------------------
#
# LSA page, "The index stops scanning the whole context", paragraphs 3-5: neighbouring keys are
# merged first (the landmarks), Ward's algorithm groups similar ones into clusters, a completed
# block's clustering is then fixed and kept as each cluster's centre plus the table of its
# positions; a query is compared with the centres only, the best clusters are expanded back to
# positions, and the start of the context and the recent window are added.  The flat variant
# scans every centre.  Readings (the page gives no constants): a "completed block" is a segment
# of seg_blocks consecutive landmarks (64 = 4096 tokens), clustered into n_clusters clusters; a
# cluster's id is its lowest member block; the candidate blocks that are not inside a completed
# segment lying wholly at or before the last candidate block are scored one by one against their
# own landmark; units are expanded in score order until K blocks are chosen.

def ward_clusters(X: np.ndarray, n_clusters: int):
    """Ward agglomerative clustering of the rows of X [n, D] into n_clusters clusters.

    Starting from singletons, the two clusters A, B whose merge increases the total
    within-cluster sum of squares the least, |A||B| / (|A|+|B|) * ||mean_A - mean_B||^2, are
    merged, until n_clusters remain.  Among equal increases the pair with the lexicographically
    smallest (id_A, id_B) is merged, a cluster's id being its lowest member row.
    Returns (members, merges): the ascending member rows of each cluster in id order, and the
    (id_A, id_B) pairs merged, in order (id_A < id_B; the merged cluster keeps id_A).
    """
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    size = np.ones(n)
    mean = X.copy()
    alive = np.ones(n, dtype=bool)
    cost = np.full((n, n), np.inf)
    iu = np.triu_indices(n, 1)
    diff = X[iu[0]] - X[iu[1]]
    cost[iu] = 0.5 * np.sum(diff * diff, axis=1)
    merges = []
    members = {i: [i] for i in range(n)}
    for _ in range(n - n_clusters):
        flat = int(np.argmin(cost))              # row-major: the first minimum is the smallest pair
        a, b = divmod(flat, n)
        mean[a] = (size[a] * mean[a] + size[b] * mean[b]) / (size[a] + size[b])
        size[a] += size[b]
        alive[b] = False
        members[a] = sorted(members[a] + members.pop(b))
        cost[b, :] = np.inf
        cost[:, b] = np.inf
        for k in np.nonzero(alive)[0]:
            if k == a:
                continue
            d = mean[a] - mean[k]
            cost[min(a, k), max(a, k)] = size[a] * size[k] / (size[a] + size[k]) * float(d @ d)
        merges.append((a, b))
    return [np.array(members[i], dtype=np.int64) for i in sorted(members)], merges


def lsa_index(L: np.ndarray, seg_blocks: int = 64, n_clusters: int = 16):
    """Flat LSA index of one (sequence, kv head): L [NB, D] landmarks (the rounded values).

    For every completed segment s (blocks s*seg_blocks .. +seg_blocks, s < NB // seg_blocks):
    Ward clusters of its landmarks; each cluster's member blocks (ascending, absolute block
    indices) and centre (the mean of its members' landmarks).  Returns a list of
    (members, centres [n_clusters, D], merges) per segment, merges in absolute block indices.
    """
    L = np.asarray(L, dtype=np.float64)
    out = []
    for s in range(L.shape[0] // seg_blocks):
        lo = s * seg_blocks
        mem, merges = ward_clusters(L[lo:lo + seg_blocks], n_clusters)
        members = [m + lo for m in mem]
        centres = np.stack([L[m].mean(axis=0) for m in members])
        out.append((members, centres, [(a + lo, b + lo) for a, b in merges]))
    return out


def lsa_select_row(qbar_c: np.ndarray, L: np.ndarray, index, c: int, topk: int, n_sink: int = 1,
                   n_local: int = 2, seg_blocks: int = 64):
    """Attended set of query block c (ascending) and the scores aligned with it, flat LSA index.

    Units: the clusters of completed segments whose blocks all lie at or before the last
    candidate block c - n_local, scored qbar . centre; and every other candidate block
    (n_sink <= j <= c - n_local) on its own, scored qbar . L_j.  Units are taken by score,
    descending (equal scores: lower id first), and expanded into their candidate blocks
    (ascending; sink blocks are attended anyway) until K blocks are chosen, the last unit cut
    short if needed.  The sink and the local window are added as in select_row.  A chosen
    block's score is its unit's score; a sink or local block's is qbar . L_j.
    """
    qbar_c = np.asarray(qbar_c, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    last = c - n_local
    n_elig = min(len(index), max(0, (last + 1) // seg_blocks))
    units = []
    for s in range(n_elig):
        members, centres, _ = index[s]
        for m, centre in zip(members, centres):
            blocks = [int(j) for j in m if j >= n_sink]
            if blocks:
                units.append((float(qbar_c @ centre), int(m[0]), blocks))
    for j in range(max(n_sink, n_elig * seg_blocks), last + 1):
        units.append((float(qbar_c @ L[j]), j, [j]))
    units.sort(key=lambda u: (-u[0], u[1]))
    chosen = {}
    for score, _, blocks in units:
        for j in blocks:
            if len(chosen) >= topk:
                break
            chosen[j] = score
        if len(chosen) >= topk:
            break
    sink = set(range(0, min(n_sink, c + 1)))
    local = set(range(max(0, c - n_local + 1), c + 1))
    A = np.array(sorted(sink | local | set(chosen)), dtype=np.int64)
    sA = np.array([chosen[j] if j in chosen else float(qbar_c @ L[j]) for j in A])
    return A, sA


# --------------------------------------------------------------------------------------
# 11. LSA tree index: beam search over groups of segments, segments, clusters
# --------------------------------------------------------------------------------------
#
# LSA page, "The index stops scanning the whole context", paragraph 5: the tree variant joins
# the clusters into a hierarchy and walks it with beam search, keeping a few branches per level,
# so a query makes a logarithmic number of comparisons.  Readings: above the Ward clusters of a
# segment sits the segment; above segments, groups of `fanout` consecutive segments; a node's
# centre is the mean of the landmarks under it.  A query uses only nodes lying wholly within its
# eligible prefix (the completed segments at or before its last candidate block); eligible
# segments not filling a whole group stand at the top level themselves.  At each level the
# `beam` best children of the kept nodes survive (equal scores: lower id first); the kept
# clusters, with the not yet clustered candidate blocks, are then expanded as in the flat index.

def lsa_tree_centres(L: np.ndarray, seg_blocks: int = 64, fanout: int = 8):
    """Centres of the segments [NS, D] and of the whole groups of `fanout` segments [NG, D]."""
    L = np.asarray(L, dtype=np.float64)
    NS = L.shape[0] // seg_blocks
    seg = np.stack([L[s * seg_blocks:(s + 1) * seg_blocks].mean(axis=0) for s in range(NS)]) \
        if NS else np.zeros((0, L.shape[1]))
    NG = NS // fanout
    grp = np.stack([seg[gi * fanout:(gi + 1) * fanout].mean(axis=0) for gi in range(NG)]) \
        if NG else np.zeros((0, L.shape[1]))
    return seg, grp


def lsa_tree_select_row(qbar_c, L, index, c: int, topk: int, n_sink: int = 1, n_local: int = 2,
                        seg_blocks: int = 64, fanout: int = 8, beam: int = 8):
    """Attended set of query block c and its scores, beam search over the tree (see above)."""
    qbar_c = np.asarray(qbar_c, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    seg_c, grp_c = lsa_tree_centres(L, seg_blocks, fanout)
    last = c - n_local
    n_elig = min(len(index), max(0, (last + 1) // seg_blocks))

    def best(cands):                      # cands: (score, id, payload); keep the beam best
        cands = sorted(cands, key=lambda x: (-x[0], x[1]))
        return cands[:beam]

    n_grp = n_elig // fanout
    top = [(float(qbar_c @ grp_c[gi]), gi * fanout * seg_blocks, ("g", gi)) for gi in range(n_grp)]
    top += [(float(qbar_c @ seg_c[s]), s * seg_blocks, ("s", s)) for s in range(n_grp * fanout, n_elig)]
    segs = []
    for _, _, (kind, i) in best(top):
        if kind == "g":
            segs += list(range(i * fanout, (i + 1) * fanout))
        else:
            segs.append(i)
    kept_segs = [p[1] for _, _, p in best([(float(qbar_c @ seg_c[s]), s * seg_blocks, ("s", s))
                                          for s in segs])]
    clusters = []
    for s in kept_segs:
        members, centres, _ = index[s]
        for m, ctr in zip(members, centres):
            blocks = [int(j) for j in m if j >= n_sink]
            if blocks:
                clusters.append((float(qbar_c @ ctr), int(m[0]), blocks))
    units = best(clusters)
    for j in range(max(n_sink, n_elig * seg_blocks), last + 1):
        units.append((float(qbar_c @ L[j]), j, [j]))
    units.sort(key=lambda u: (-u[0], u[1]))
    chosen = {}
    for score, _, blocks in units:
        for j in blocks:
            if len(chosen) >= topk:
                break
            chosen[j] = score
        if len(chosen) >= topk:
            break
    sink = set(range(0, min(n_sink, c + 1)))
    local = set(range(max(0, c - n_local + 1), c + 1))
    A = np.array(sorted(sink | local | set(chosen)), dtype=np.int64)
    sA = np.array([chosen[j] if j in chosen else float(qbar_c @ L[j]) for j in A])
    return A, sA


# --------------------------------------------------------------------------------------
# 12. decode-time maintenance
# --------------------------------------------------------------------------------------
#
# LSA page, "The index stops scanning the whole context", paragraph 3: keys are pooled per block
# and a block's clusters are computed once the block is complete and then kept.  A landmark is a
# function of its own block's keys only, so appending tokens changes only the blocks that hold
# them; a completed segment's clustering never changes.

def update_landmarks(lm, k, n_new: int, dtype: str, block: int = BLOCK) -> np.ndarray:
    """lm [B,H,NB,D] with the blocks holding the last n_new tokens of k [B,H,T,D] recomputed as
    block means (rounded to dtype); every other block keeps its value from lm."""
    B, H, T, D = k.shape
    out = np.array(lm, dtype=np.float64, copy=True)
    for j in range(max(T - n_new, 0) // block, n_blocks(T, block)):
        lo, hi = j * block, min((j + 1) * block, T)
        out[:, :, j, :] = round_to_dtype(k[:, :, lo:hi, :].mean(axis=2), dtype)
    return out


def update_landmarks_paged(lm, k_pool, page_table, seq_lens, n_new: int, dtype: str,
                           block: int = BLOCK) -> np.ndarray:
    """Paged layout: sequence b's blocks holding its last n_new tokens are recomputed from its
    pages; its other blocks (and blocks past its end) keep their value from lm [B,Hkv,NB,D]."""
    out = np.array(lm, dtype=np.float64, copy=True)
    for b, L in enumerate(seq_lens):
        L = int(L)
        for j in range(max(L - n_new, 0) // block, (L - 1) // block + 1):
            n = min(block, L - j * block)
            out[b, :, j, :] = round_to_dtype(k_pool[int(page_table[b][j]), :, :n, :].mean(axis=1),
                                             dtype)
    return out


def lsa_update_index(index, L: np.ndarray, first_segment: int, seg_blocks: int = 64,
                     n_clusters: int = 16):
    """The index of lsa_index after the segments first_segment .. NS-1 completed: the entries of
    the earlier segments are kept as they are (the same objects), the new segments clustered."""
    L = np.asarray(L, dtype=np.float64)
    fresh = lsa_index(L, seg_blocks, n_clusters)
    return list(index[:first_segment]) + fresh[first_segment:]

