"""Plain, slow, fp64 CPU oracle for exact scaled dot-product attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the package smoke check and the
bench's CPU-baseline leg use it.  It shares no code, constant or helper with
the HIP library; the only thing both sides see is the seeded input tensors.

What it computes is the plain definition, written out with one library
primitive (a dense matmul) per contraction and nothing fused, blocked or
reordered:

* scores     s_ij = scale * sum_d q[i,d] * k[j,d]
  (tensai autograd guide, section "Attention の組み立て": q.MatMul(k.T()) then
  Scale(1/sqrt(headDim)); HOF Flash Attention essay, section 4 "カーネル":
  q.dot(k.t()) divided by a square root).  The scale is an argument; the
  essay's width-based scale and the guide's headDim-based scale are both
  particular values of it.
* mask       z_ij = s_ij + mask_ij, mask 0 where key j is visible to query i
  and -inf elsewhere, added after scaling (tensai guide, same section: the
  constant (1,1,seq,seq) mask is 0 on and below the diagonal, -inf above, and
  broadcasts over batch and head; "ブロードキャスト" section).  Key padding
  hides keys j >= key_lens[b] for every query of batch b.
* softmax    a_ij = exp(z_ij - m_i) / sum_j exp(z_ij - m_i), m_i = max_j z_ij,
  over the last (key) axis (tensai guide, section "演算": Softmax acts on the
  final axis; HOF essay section 4: exp of the scores divided by the row sums
  gives a row-stochastic A).  Subtracting the row max is the one departure
  from the essay's printed kernel, which exponentiates raw scores; the two
  agree exactly in real arithmetic because softmax is shift invariant.
* output     o_i = sum_j a_ij v_j   (HOF essay section 4: weights.dot(v)).
* lse        lse_i = m_i + ln(sum_j exp(z_ij - m_i))  (the log of the softmax
  denominator, used by the split-KV partials); -inf for a row with no
  visible key (the log of an empty sum).
* widths     q and k share the key width D, v has its own width Dv and the
  output has Dv columns (ruDNN user guide section 9: K is [.., Hkv, D], V is
  [.., Hkv, Dv], the output [.., Hq, Dv], with D and Dv each in 1..=1024);
  every function below takes v of any width Dv >= 1.
* head map   query head h reads K/V head floor(h / (Hq / Hkv)) (grouped K/V,
  ruDNN user guide section 9 "ページ化アテンションと MLA": Hq must be divisible
  by Hkv; contiguous groups is the reading taken).
* bias       a general additive mask [B or 1, Hq or 1, Sq, Sk] added to the
  scaled scores next to the 0 / -inf masks (tensai guide, "Attention の
  組み立て": the scores are scaled and then Add(mask) with a mask tensor that
  broadcasts over its size-1 batch and head axes); -inf entries hide keys.
* block      the multi-head attention block around it (tensai guide,
  "Attention の組み立て"): q, k, v = heads(x . w) for w in wq, wk, wv, where
  heads reshapes (batch, seq, model) to (batch, seq, head, headDim) and swaps
  seq and head; the attention above; y = heads^-1(o) . wo.
* split-KV   partial attention over disjoint key ranges, each with its own lse,
  and the log-sum-exp merge of those partials (ruDNN user guide section 9:
  history split into 2..=32 pieces, partial statistics and merge in FP32).
* backward   gradients of a loss L through O = softmax(S) V, S = scale Q K^T +
  mask, given dO = dL/dO (ruDNN user guide section 11: the attention backward
  returns dq, dk, dv and recomputes the probabilities instead of storing the
  score matrix; tensai guide, the block step's backward).  With P the row
  softmax: dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dO * O)) (the
  softmax Jacobian applied row by row); dQ = scale dS K; dK = scale dS^T Q.
  Grouped K/V: a K/V head's dK, dV sum the contributions of its query heads.
  A row with no visible key has no defined output and contributes nothing
  (its dQ row is 0).
* paged      packed queries [queries, Hq, D] over a physical K/V page cache
  [pages, page_size, Hkv, D] (ruDNN user guide section 9): query t belongs to
  sequence query_seq[t] at zero-based absolute position query_pos[t]; the
  sequence's logical key j (j < seq_lens[s]) sits in physical page
  block_tables[s][j // page_size], slot j % page_size; with the causal flag
  key j is visible only when j <= query_pos[t] (absolute positions, so a
  chunk of new queries at the end of a sequence is aligned bottom-right).
  Its backward (ruDNN user guide section 11) gives dq and the gradients of
  the cache slots: each logical key's contribution is added into the slot it
  sits in, unreached slots get 0.

A row with no visible key has 0/0 weights and yields NaN, the literal result
of the essay's normalisation (ruDNN user guide section 4 likewise keeps NaN
for rows with no finite logit).

Every function here is pinned by tests/test_oracle.py against closed forms,
invariants, special cases and brute force; none is "parity unpinned".
"""

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_KEY_PADDING = 2


def _check_shapes(q, k, v):
    """Sizes of q [B,Hq,Sq,D], k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv]: (B, Hq, Hkv,
    Sk, D, Dv)."""
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D (batch, head, seq, headDim)")
    B, Hq, _, D = q.shape
    Bk, Hkv, Sk, Dk = k.shape
    if Bk != B or Dk != D or v.shape[:3] != k.shape[:3] or v.shape[3] < 1:
        raise ValueError("inconsistent q/k/v shapes %s %s %s" % (q.shape, k.shape, v.shape))
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Sk, D, v.shape[3]


def visible_rows(mask_kind, rows, Sk, key_len):
    """Boolean [len(rows), Sk]: True where key j is visible to query row i.

    rows are query positions.  Causal: j <= i (tensai guide, "Attention の組み立て":
    0 on and below the diagonal).  Key padding: j < key_len.
    """
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Sk, dtype=np.int64)[None, :]
    vis = np.ones((rows.shape[0], Sk), dtype=bool)
    if mask_kind & MASK_CAUSAL:
        vis &= j <= rows[:, None]
    if mask_kind & MASK_KEY_PADDING:
        vis &= j < int(key_len)
    return vis


def attend(qrows, kh, vh, scale, vis, bias=None):
    """Attention of query rows over one K/V head, by the definition.

    qrows [n, D], kh and vh [Sk, D], vis [n, Sk] bool, bias None or [n, Sk]
    (an additive mask, added to the scaled scores like the 0 / -inf one).
    Returns (o [n, D], lse [n], a [n, Sk]) in fp64.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    s = float(scale) * (qrows @ kh.T)          # scale first ...
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)   # ... then the additive masks:
    z = np.where(vis, s, -np.inf)              # the bias, and the 0 / -inf mask
    with np.errstate(invalid="ignore", divide="ignore"):
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)                      # exp(-inf) = 0 on hidden keys
        l = e.sum(axis=1, keepdims=True)
        a = e / l                              # row-stochastic weights
        o = a @ vh
        # ln of the denominator; a row with no visible key has the empty sum,
        # ln 0 = -inf (the max-shifted form would give NaN there)
        lse = np.where(np.isneginf(m[:, 0]), -np.inf, (m + np.log(l))[:, 0])
    return o, lse, a


def bias_slice(bias, b, h):
    """The [Sq, Sk] additive mask of (batch b, query head h) from a bias of
    shape [B or 1, Hq or 1, Sq, Sk] (a size-1 axis broadcasts, as the tensai
    guide's (1, 1, seq, seq) mask does over batch and heads)."""
    if bias is None:
        return None
    return bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0]


def _check_bias(bias, B, Hq, Sq, Sk):
    if bias is None:
        return None
    bias = np.asarray(bias)
    if (bias.ndim != 4 or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, Hq)
            or bias.shape[2:] != (Sq, Sk)):
        raise ValueError("bias must be [B or 1, Hq or 1, Sq, Sk], got %s" % (bias.shape,))
    return bias


def sdpa_forward(q, k, v, scale, mask_kind=MASK_NONE, key_lens=None,
                 return_lse=False, return_probs=False, bias=None):
    """Full forward O = softmax(Q K^T * scale + mask) V for every (b, h, i).

    q [B,Hq,Sq,D], k and v [B,Hkv,Sk,D]; key_lens [B] when mask_kind has the
    key-padding bit.  The causal mask is defined for square attention only
    (the tensai guide's (seq, seq) mask), so causal with Sq != Sk is an error.
    bias: optional general additive mask [B or 1, Hq or 1, Sq, Sk] added to
    the scaled scores (the tensai guide's Add(mask) with any mask tensor),
    together with the causal / padding masks.
    Returns o (fp64), plus lse [B,Hq,Sq] and/or probs [B,Hq,Sq,Sk] on request.
    """
    q = np.asarray(q)
    B, Hq, Hkv, Sk, D, Dv = _check_shapes(q, np.asarray(k), np.asarray(v))
    Sq = q.shape[2]
    if mask_kind & MASK_CAUSAL and Sq != Sk:
        raise ValueError("causal mask needs Sq == Sk")
    if bool(mask_kind & MASK_KEY_PADDING) != (key_lens is not None):
        raise ValueError("key_lens is given exactly when the key-padding bit is set")
    bias = _check_bias(bias, B, Hq, Sq, Sk)
    G = Hq // Hkv
    o = np.empty((B, Hq, Sq, Dv), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)
    probs = np.empty((B, Hq, Sq, Sk), dtype=np.float64) if return_probs else None
    rows = np.arange(Sq)
    for b in range(B):
        vis = visible_rows(mask_kind, rows, Sk, key_lens[b] if key_lens is not None else 0)
        for h in range(Hq):
            g = h // G
            o[b, h], lse[b, h], a = attend(q[b, h], k[b, g], v[b, g], scale, vis,
                                           bias_slice(bias, b, h))
            if return_probs:
                probs[b, h] = a
    out = [o]
    if return_lse:
        out.append(lse)
    if return_probs:
        out.append(probs)
    return out[0] if len(out) == 1 else tuple(out)


def sdpa_forward_rows(q, k, v, scale, mask_kind, key_lens, index, bias=None):
    """Selected output rows only: index is an int array [n, 3] of (b, h, i).

    Same definition as sdpa_forward, evaluated only for the listed query rows
    (grouped by head) so that it scales to full-size workloads.  q, k, v (and
    bias, [B or 1, Hq or 1, Sq, Sk]) may be any array-likes indexable as
    [b, h] (only the needed heads are read).
    Returns (o [n, Dv], lse [n]) in the order of index (v is [B, Hkv, Sk, Dv]).
    """
    B, Hq, _ = q.shape[0], q.shape[1], q.shape[2]
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if mask_kind & MASK_CAUSAL and q.shape[2] != Sk:
        raise ValueError("causal mask needs Sq == Sk")
    G = Hq // Hkv
    index = np.asarray(index, dtype=np.int64).reshape(-1, 3)
    o = np.empty((index.shape[0], Dv), dtype=np.float64)
    lse = np.empty(index.shape[0], dtype=np.float64)
    heads = {}
    for n, (b, h, i) in enumerate(index):
        heads.setdefault((int(b), int(h)), []).append((n, int(i)))
    for (b, h), items in heads.items():
        pos = np.array([n for n, _ in items])
        rows = np.array([i for _, i in items])
        klen = key_lens[b] if key_lens is not None else 0
        vis = visible_rows(mask_kind, rows, Sk, klen)
        g = h // G
        qh = np.asarray(q[b, h])
        bh = None
        if bias is not None:
            bh = np.asarray(bias[b if bias.shape[0] > 1 else 0, h if bias.shape[1] > 1 else 0])[rows]
        o[pos], lse[pos], _ = attend(qh[rows], k[b, g], v[b, g], scale, vis, bh)
    return o, lse


def sdpa_decode(q, k, v, scale, key_lens=None):
    """Single-query decode: the forward with Sq = 1 and no causal mask.

    Every cached key is visible except those past key_lens[b] when given.
    """
    kind = MASK_KEY_PADDING if key_lens is not None else MASK_NONE
    return sdpa_forward(q, k, v, scale, kind, key_lens)


def split_ranges(Sk, num_splits):
    """Key range [lo, hi) of each split: chunks of ceil(Sk / num_splits) keys."""
    chunk = -(-Sk // num_splits)
    return [(min(s * chunk, Sk), min((s + 1) * chunk, Sk)) for s in range(num_splits)]


def decode_split_partials(q, k, v, scale, key_lens, num_splits):
    """Per-split partial attention for decode (q [B,Hq,1,D]).

    Split s attends only to its key range (intersected with the visible keys)
    and yields a normalised partial output and its log-sum-exp.  A split with
    no visible key contributes o = 0 and lse = -inf (an empty softmax
    denominator).  Returns (o_part [B,Hq,n,D], lse_part [B,Hq,n]).
    """
    B, Hq, Hkv, Sk, D, Dv = _check_shapes(q, k, v)
    G = Hq // Hkv
    o_part = np.zeros((B, Hq, num_splits, Dv), dtype=np.float64)
    lse_part = np.full((B, Hq, num_splits), -np.inf, dtype=np.float64)
    for b in range(B):
        vis_all = visible_rows(MASK_KEY_PADDING if key_lens is not None else MASK_NONE,
                               [0], Sk, key_lens[b] if key_lens is not None else 0)
        for s, (lo, hi) in enumerate(split_ranges(Sk, num_splits)):
            vis = vis_all[:, lo:hi]
            if not vis.any():
                continue
            for h in range(Hq):
                g = h // G
                on, ln, _ = attend(q[b, h, 0:1], k[b, g, lo:hi], v[b, g, lo:hi], scale, vis)
                o_part[b, h, s], lse_part[b, h, s] = on[0], ln[0]
    return o_part, lse_part


def merge_partials(o_part, lse_part):
    """Log-sum-exp merge of split partials over the split axis.

    o = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M), M = max_s lse_s.
    o_part [..., n, D], lse_part [..., n]; returns (o [..., D], lse [...]).
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        M = lse_part.max(axis=-1, keepdims=True)
        w = np.exp(lse_part - M)
        den = w.sum(axis=-1, keepdims=True)
        o = (w[..., None] * o_part).sum(axis=-2) / den
        lse = (M + np.log(den))[..., 0]
    return o, lse


def sdpa_backward(q, k, v, dout, scale, mask_kind=MASK_NONE, key_lens=None, bias=None,
                  return_dbias=False):
    """dQ, dK, dV (and the bias gradient) of L with dL/dO = dout, by the definition (fp64).

    q [B,Hq,Sq,D], dout [B,Hq,Sq,Dv]; k [B,Hkv,Sk,D], v [B,Hkv,Sk,Dv]; bias None or [B or 1, Hq or 1,
    Sq, Sk], added to the scaled scores as in sdpa_forward.  Per (b, h): P is
    the row softmax of the masked biased scaled scores (hidden keys get
    exactly 0), O = P V, then dV = P^T dO, dP = dO V^T, dS = P * (dP -
    rowsum(dO * O)), dQ = scale dS K, dK = scale dS^T Q; dK and dV of a K/V
    head sum over its Hq/Hkv query heads.  dS is the gradient of the biased
    scores, so the gradient of a [B, Hq, Sq, Sk] bias is dS itself (a
    broadcast bias would sum it over its size-1 axes).  Rows with no visible
    key of finite weight (lse = -inf) contribute nothing.  Returns (dq, dk,
    dv), or (dq, dk, dv, dbias [B, Hq, Sq, Sk]) with return_dbias.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Hkv, Sk, D, Dv = _check_shapes(q, k, v)
    Sq = q.shape[2]
    if mask_kind & MASK_CAUSAL and Sq != Sk:
        raise ValueError("causal mask needs Sq == Sk")
    if dout.shape != (B, Hq, Sq, Dv):
        raise ValueError("dout must be [B, Hq, Sq, Dv]")
    bias = _check_bias(bias, B, Hq, Sq, Sk)
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dbias = np.zeros((B, Hq, Sq, Sk)) if return_dbias else None
    rows = np.arange(Sq)
    for b in range(B):
        vis = visible_rows(mask_kind, rows, Sk, key_lens[b] if key_lens is not None else 0)
        for h in range(Hq):
            g = h // G
            _, lse, p = attend(q[b, h], k[b, g], v[b, g], scale, vis, bias_slice(bias, b, h))
            live = np.isfinite(lse)            # rows with a visible key of finite weight
            p = np.where(live[:, None], p, 0.0)
            do = np.where(live[:, None], dout[b, h], 0.0)
            o = p @ v[b, g]
            dv[b, g] += p.T @ do
            dp = do @ v[b, g].T
            ds = p * (dp - (do * o).sum(axis=1, keepdims=True))
            dq[b, h] = float(scale) * (ds @ k[b, g])
            dk[b, g] += float(scale) * (ds.T @ q[b, h])
            if dbias is not None:
                dbias[b, h] = ds
    return (dq, dk, dv, dbias) if return_dbias else (dq, dk, dv)


def split_heads(t, n_heads):
    """(batch, seq, model) -> (batch, head, seq, headDim): reshape to
    (batch, seq, head, headDim), then swap the seq and head axes (tensai guide,
    "Attention の組み立て", the heads helper)."""
    B, S, M = t.shape
    return t.reshape(B, S, n_heads, M // n_heads).transpose(0, 2, 1, 3)


def merge_heads(t):
    """(batch, head, seq, headDim) -> (batch, seq, model): the inverse of split_heads."""
    B, H, S, hd = t.shape
    return t.transpose(0, 2, 1, 3).reshape(B, S, H * hd)


def block_forward(x, wq, wk, wv, wo, n_heads, scale=None, mask_kind=MASK_NONE, key_lens=None):
    """Multi-head attention block of the tensai guide ("Attention の組み立て").

    x [B, S, model]; wq, wk, wv, wo [model, model] (x is multiplied on the
    left: x . w).  q, k, v = split_heads(x . w{q,k,v}); the attention of
    sdpa_forward (scale defaults to 1 / sqrt(headDim)); y = merge_heads(o) . wo.
    Returns y [B, S, model] in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    B, S, M = x.shape
    if M % n_heads != 0:
        raise ValueError("model width must be a multiple of the head count")
    for w in (wq, wk, wv, wo):
        if w.shape != (M, M):
            raise ValueError("weights must be [model, model]")
    if scale is None:
        scale = 1.0 / np.sqrt(M // n_heads)
    q = split_heads(x @ wq, n_heads)
    k = split_heads(x @ wk, n_heads)
    v = split_heads(x @ wv, n_heads)
    o = sdpa_forward(q, k, v, scale, mask_kind, key_lens)
    return merge_heads(o) @ wo


def block_forward_rows(x, wq, wk, wv, wo, n_heads, rows, scale=None, mask_kind=MASK_NONE,
                       key_lens=None):
    """Selected rows of block_forward: rows is an int array [n, 2] of (b, s).

    Same definition as block_forward, with the projections computed only for
    the batches that hold a listed row and the attention only for the listed
    query positions (sdpa_forward_rows), so that it scales to full-size
    workloads.  Returns y [n, model] in fp64, in the order of rows.
    """
    B, S, M = x.shape
    if M % n_heads != 0:
        raise ValueError("model width must be a multiple of the head count")
    if scale is None:
        scale = 1.0 / np.sqrt(M // n_heads)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    y = np.empty((rows.shape[0], M), dtype=np.float64)
    for b in np.unique(rows[:, 0]):
        sel = np.nonzero(rows[:, 0] == b)[0]
        xb = np.asarray(x[b:b + 1], dtype=np.float64)
        q = split_heads(xb @ wq, n_heads)
        k = split_heads(xb @ wk, n_heads)
        v = split_heads(xb @ wv, n_heads)
        index = np.array([(0, h, rows[n, 1]) for n in sel for h in range(n_heads)])
        lens = None if key_lens is None else np.asarray(key_lens)[b:b + 1]
        o, _ = sdpa_forward_rows(q, k, v, scale, mask_kind, lens, index)
        # o holds, per listed row, its heads in order: concatenated they are
        # the merged (seq, model) row
        y[sel] = o.reshape(sel.size, M) @ wo
    return y


def paged_gather(cache, table_row, length, page_size):
    """Logical rows 0..length-1 of one sequence read through its page table.

    cache [pages, page_size, Hkv, D]; logical row j is physical page
    table_row[j // page_size], slot j % page_size (ruDNN user guide section 9:
    the kernels read the physical cache pages directly).  Returns
    [length, Hkv, D].
    """
    j = np.arange(int(length), dtype=np.int64)
    table_row = np.asarray(table_row, dtype=np.int64)
    return np.asarray(cache)[table_row[j // page_size], j % page_size]


def paged_attention(q, k_cache, v_cache, block_tables, seq_lens, query_seq, query_pos,
                    scale, causal):
    """Packed paged attention (ruDNN user guide section 9).

    q [queries, Hq, D]; k_cache [pages, page_size, Hkv, D]; v_cache [pages,
    page_size, Hkv, Dv];
    block_tables [num_seqs, max_pages_per_seq]; seq_lens [num_seqs];
    query_seq, query_pos [queries].  Query t (sequence s = query_seq[t],
    position p = query_pos[t]) attends to keys j < seq_lens[s] of its own
    sequence, and with causal only to j <= p.  Query head h reads K/V head
    h // (Hq / Hkv).  Returns o [queries, Hq, Dv] in fp64 (NaN rows where no key
    is visible).
    """
    q = np.asarray(q)
    nq, Hq, D = q.shape
    pages, page_size, Hkv, Dk = np.asarray(k_cache).shape
    vshape = np.asarray(v_cache).shape
    if Dk != D or len(vshape) != 4 or vshape[:3] != (pages, page_size, Hkv) or vshape[3] < 1:
        raise ValueError("inconsistent q / cache shapes")
    Dv = vshape[3]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.empty((nq, Hq, Dv), dtype=np.float64)
    for t in range(nq):
        s_id, pos = int(query_seq[t]), int(query_pos[t])
        length = int(seq_lens[s_id])
        ks = paged_gather(k_cache, block_tables[s_id], length, page_size)
        vs = paged_gather(v_cache, block_tables[s_id], length, page_size)
        j = np.arange(length, dtype=np.int64)
        vis = np.ones((1, length), dtype=bool)
        if causal:
            vis &= (j <= pos)[None, :]
        for h in range(Hq):
            g = h // G
            o[t, h] = attend(q[t, h:h + 1], ks[:, g], vs[:, g], scale, vis)[0][0]
    return o


def paged_attention_backward(q, k_cache, v_cache, dout, block_tables, seq_lens, query_seq,
                             query_pos, scale, causal):
    """Gradients of L with dL/dO = dout through paged_attention (ruDNN user
    guide section 11: the paged plan's attention backward returns dq and the
    history gradients dk, dv, recomputing the probabilities).

    q [queries, Hq, D], dout [queries, Hq, Dv]; k_cache [pages, page_size,
    Hkv, D], v_cache [.., Dv].  Per query t and head h, with ks, vs the keys
    and values its sequence reaches through its page table (paged_gather) and
    p the softmax of the visible scaled scores: dv_j += p_j dout, dp_j =
    dout . vs_j, ds_j = p_j (dp_j - dout . o), dq = scale sum_j ds_j ks_j,
    dk_j += scale ds_j q.  The cache gradients are added into the physical
    slot each logical key j sits in (a slot reached twice gets both
    contributions); slots no visible key reaches get 0.  Returns (dq,
    dk_cache, dv_cache) in fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    nq, Hq, D = q.shape
    pages, page_size, Hkv, Dk = k_cache.shape
    Dv = v_cache.shape[3]
    if Dk != D or v_cache.shape[:3] != k_cache.shape[:3] or dout.shape != (nq, Hq, Dv):
        raise ValueError("inconsistent q / cache / dout shapes")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_cache)
    dv = np.zeros_like(v_cache)
    for t in range(nq):
        s_id, pos = int(query_seq[t]), int(query_pos[t])
        length = int(seq_lens[s_id])
        table_row = np.asarray(block_tables[s_id], dtype=np.int64)
        j = np.arange(length, dtype=np.int64)
        page, slot = table_row[j // page_size], j % page_size
        ks = k_cache[page, slot]               # [length, Hkv, D]
        vs = v_cache[page, slot]
        vis = np.ones((1, length), dtype=bool)
        if causal:
            vis &= (j <= pos)[None, :]
        for h in range(Hq):
            g = h // G
            o, lse, p = attend(q[t, h:h + 1], ks[:, g], vs[:, g], scale, vis)
            if not np.isfinite(lse[0]):
                continue                       # no visible key: no output, no gradient
            p = p[0]
            do = dout[t, h]
            dp = vs[:, g] @ do
            ds = p * (dp - float(do @ o[0]))
            dq[t, h] = float(scale) * (ds @ ks[:, g])
            np.add.at(dk, (page, slot, g), float(scale) * ds[:, None] * q[t, h][None, :])
            np.add.at(dv, (page, slot, g), p[:, None] * do[None, :])
    return dq, dk, dv


def chunk_positions(cu_seqlens_q, seq_lens):
    """Sequence and absolute position of every packed query of a prefill chunk.

    Queries cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 belong to sequence s and are
    its last n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s] tokens: query i of the
    sequence sits at position seq_lens[s] - n_s + i (the new tokens are
    appended after the cached ones, ruDNN user guide section 9: positions are
    zero-based absolute positions within each sequence).  Returns
    (query_seq, query_pos) for paged_attention.
    """
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    qs, qp = [], []
    for s in range(len(cu) - 1):
        n = int(cu[s + 1] - cu[s])
        qs.extend([s] * n)
        qp.extend(int(seq_lens[s]) - n + i for i in range(n))
    return np.array(qs, dtype=np.int64), np.array(qp, dtype=np.int64)


__all__ = [
    "MASK_NONE", "MASK_CAUSAL", "MASK_KEY_PADDING", "visible_rows", "attend",
    "sdpa_forward", "sdpa_forward_rows", "sdpa_decode", "split_ranges",
    "decode_split_partials", "merge_partials", "paged_gather", "paged_attention",
    "chunk_positions", "sdpa_backward", "bias_slice", "split_heads", "merge_heads",
    "block_forward", "block_forward_rows", "paged_attention_backward",
]
