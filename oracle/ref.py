"""Plain numpy forms of the Gated DeltaNet hot path, for small cases.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module; it exists to pin the fp64 C oracle (``gdn_oracle.c``) to things other
than itself.  Every function is fp64 and loops in plain Python where the
definition is a loop, so it is meant for tiny inputs only.

Pages cited:
  * flash-linear-attention ``fla/ops/cp/context.py`` -- ``get_cp_cu_seqlens``.
  * hyper-parallel ``linear_attention_context_parallel.py`` --
    ``_causal_conv1d_with_cp_halo``, ``_l2norm_torch``,
    ``_prepare_gdn_chunks_for_summary``, ``_run_prepared_gdn_chunks``,
    ``_compute_gdn_state_summary_from_prepared``,
    ``_merge_gdn_prefix_state_summaries_torch``, ``_apply_gdn_state_summary``.
  * h3-blackwell-runtime ``distributed.py`` -- ``localize_segments``.
"""
from __future__ import annotations

import numpy as np

L2NORM_EPS = 1e-6


# --------------------------------------------------------------------------
# Localisation
# --------------------------------------------------------------------------
def localize_p1(cu, world_size, rank, conv_k):
    """fla ``get_cp_cu_seqlens`` restated with numpy (steps 2-5 of the page).

    Returns (local_cu int64 array, meta dict).  The shard is
    [part_len*rank, part_len*(rank+1)) with part_len = total // world_size;
    two sorted searches select the overlapping sequences; their boundaries are
    clamped to the shard, rebased and de-duplicated.
    """
    cu = np.asarray(cu, dtype=np.int64)
    total = int(cu[-1])
    part_len = total // world_size
    rank_start = part_len * rank
    rank_end = rank_start + part_len
    start_idx = int(np.searchsorted(cu[1:], rank_start, side="right"))
    end_idx = int(np.searchsorted(cu[:-1], rank_end, side="left"))
    sub = np.clip(cu[start_idx:end_idx + 1], rank_start, rank_end) - rank_start
    keep = np.ones(len(sub), dtype=bool)
    keep[1:] = sub[1:] != sub[:-1]
    local = sub[keep]
    first_start = int(cu[start_idx])
    last_end = int(cu[end_idx])
    pre_conv = max(0, rank_start - first_start)
    first_rank = first_start // part_len
    last_rank = (last_end - 1) // part_len
    meta = dict(
        rank_start=rank_start,
        rank_end=rank_end,
        num_local_seqs=len(local) - 1,
        first_seq_global_idx=start_idx,
        is_first_rank=int(rank == first_rank),
        is_last_rank=int(rank == last_rank),
        pre_num_ranks=rank - first_rank,
        post_num_ranks=last_rank - rank,
        pre_num_conv_tokens=pre_conv,
        n_halo=min(max(conv_k - 1, 0), pre_conv),
    )
    return local, meta


def localize_bruteforce(cu, world_size, rank, conv_k):
    """Per-token enumeration of the same quantities, no searching.

    Every global token t is owned by rank t // part_len.  The local pieces
    are each sequence's tokens owned by ``rank`` with empty pieces dropped
    (the clip rule of h3-blackwell-runtime ``localize_segments``).  The first
    (last) local sequence is the one holding the shard's first (last) token;
    its first (last) owner is the owner of its first (last) token.
    """
    cu = [int(c) for c in cu]
    total = cu[-1]
    part_len = total // world_size
    owner = [t // part_len for t in range(total)]
    seq_of = []
    for n in range(len(cu) - 1):
        seq_of += [n] * (cu[n + 1] - cu[n])
    mine = [t for t in range(total) if owner[t] == rank]
    pieces = []
    for n in range(len(cu) - 1):
        toks = [t for t in range(cu[n], cu[n + 1]) if owner[t] == rank]
        if toks:
            pieces.append((n, len(toks)))
    local = [0]
    for _, ln in pieces:
        local.append(local[-1] + ln)
    first_tok, last_tok = mine[0], mine[-1]
    n_first, n_last = seq_of[first_tok], seq_of[last_tok]
    first_owner = owner[cu[n_first]]
    last_owner = owner[cu[n_last + 1] - 1]
    pre_conv = first_tok - cu[n_first]
    meta = dict(
        rank_start=first_tok,
        rank_end=last_tok + 1,
        num_local_seqs=len(pieces),
        first_seq_global_idx=n_first,
        is_first_rank=int(rank == first_owner),
        is_last_rank=int(rank == last_owner),
        pre_num_ranks=rank - first_owner,
        post_num_ranks=last_owner - rank,
        pre_num_conv_tokens=pre_conv,
        n_halo=min(max(conv_k - 1, 0), pre_conv),
    )
    return np.asarray(local, dtype=np.int64), meta


# --------------------------------------------------------------------------
# Conv
# --------------------------------------------------------------------------
def silu(z):
    return z / (1.0 + np.exp(-z))


def conv1d_silu(x, w, bias, halo, n_halo, cu):
    """Causal depthwise conv (cross-correlation: w[:, K-1] multiplies the
    current token) + SiLU per sequence.  Sequence 0 sees the last n_halo rows
    of ``halo`` before its start; every other position before a sequence start
    is zero (hyper-parallel ``_causal_conv1d_with_cp_halo``)."""
    x = np.asarray(x, np.float64)
    T, C = x.shape
    K = w.shape[1]
    y = np.zeros_like(x)
    for n in range(len(cu) - 1):
        s, e = int(cu[n]), int(cu[n + 1])
        pad = np.zeros((K - 1, C))
        if n == 0 and halo is not None and n_halo > 0:
            pad[K - 1 - n_halo:] = halo[K - 1 - n_halo:]
        xs = np.concatenate([pad, x[s:e]], axis=0)
        for t in range(e - s):
            z = (xs[t:t + K] * w.T).sum(axis=0)
            if bias is not None:
                z = z + bias
            y[s + t] = silu(z)
    return y


# --------------------------------------------------------------------------
# Gated delta rule
# --------------------------------------------------------------------------
def l2norm(x):
    """hyper-parallel ``_l2norm_torch``: x * rsqrt(sum(x^2) + 1e-6)."""
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + L2NORM_EPS)


def _prep(q, k, scale, use_l2norm):
    if use_l2norm:
        q, k = l2norm(q), l2norm(k)
    return q * scale, k


def gdn_recurrent(q, k, v, g, beta, h0, cu, scale, use_l2norm=True):
    """Token recurrence, state [dk, dv]: decay, delta update, readout.

    q, k [T,Hk,dk]; v [T,Hv,dv]; g, beta [T,Hv]; h0 [N,Hv,dk,dv] or None.
    Returns o [T,Hv,dv], ht [N,Hv,dk,dv]."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    qh, kh = _prep(q, k, scale, use_l2norm)
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    ht = np.zeros((N, Hv, dk, dv))
    for n in range(N):
        for h in range(Hv):
            a = h // grp
            S = np.zeros((dk, dv)) if h0 is None else h0[n, h].copy()
            for t in range(int(cu[n]), int(cu[n + 1])):
                S = np.exp(g[t, h]) * S
                u = beta[t, h] * (v[t, h] - S.T @ kh[t, a])
                S = S + np.outer(kh[t, a], u)
                o[t, h] = S.T @ qh[t, a]
            ht[n, h] = S
    return o, ht


def gdn_bruteforce(q, k, v, g, beta, h0, cu, scale, use_l2norm=True):
    """Dense transition products instead of a recurrence.

    Token t maps the state by S -> A_t S + B_t with
    A_t = e^{g_t} (I - beta_t k_t k_t^T) and B_t = beta_t k_t v_t^T, so
    S_t = (A_t ... A_s) h0 + sum_r (A_t ... A_{r+1}) B_r.  Each S_t is built
    from scratch from these products."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    qh, kh = _prep(q, k, scale, use_l2norm)
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    ht = np.zeros((N, Hv, dk, dv))
    I = np.eye(dk)
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(Hv):
            a = h // grp
            A = [np.exp(g[t, h]) * (I - beta[t, h] * np.outer(kh[t, a], kh[t, a])) for t in range(s, e)]
            B = [beta[t, h] * np.outer(kh[t, a], v[t, h]) for t in range(s, e)]
            init = np.zeros((dk, dv)) if h0 is None else h0[n, h]
            for i in range(e - s):
                prod = I.copy()
                for r in range(i, -1, -1):
                    prod = prod @ A[r]
                St = prod @ init
                for r in range(i + 1):
                    P = I.copy()
                    for m in range(i, r, -1):
                        P = P @ A[m]
                    St = St + P @ B[r]
                o[s + i, h] = St.T @ qh[s + i, a]
                if i == e - s - 1:
                    ht[n, h] = St
            if e == s:
                ht[n, h] = init
    return o, ht


def _chunk_prepare(qh, kh, vv, gg, bb, C):
    """The page's chunk preparation for one sequence and head, rows padded
    with zeros to a multiple of C (hyper-parallel
    ``_prepare_gdn_chunks_for_summary``):  in-chunk cumsum G of g; decay
    matrix Gamma_ij = exp(G_i - G_j) on and below the diagonal;
    L = strict-lower(diag(beta) K K^T o Gamma); T = (I + L)^-1 by forward
    substitution; u = T diag(beta) V; w = T diag(beta e^G) K."""
    L_ = qh.shape[0]
    pad = (-L_) % C
    def padr(x):
        return np.concatenate([x, np.zeros((pad,) + x.shape[1:])], axis=0)
    qh, kh, vv, gg, bb = map(padr, (qh, kh, vv, gg, bb))
    nch = qh.shape[0] // C
    out = []
    for c in range(nch):
        sl = slice(c * C, (c + 1) * C)
        q_c, k_c, v_c, b_c = qh[sl], kh[sl], vv[sl], bb[sl]
        G = np.cumsum(gg[sl])
        diff = G[:, None] - G[None, :]
        lower = np.tril(np.ones((C, C), dtype=bool))
        Gam = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        Lm = np.tril(b_c[:, None] * (k_c @ k_c.T) * Gam, -1)
        # forward substitution for the rows of (I + L)^-1, row by row
        Tm = np.zeros((C, C))
        for i in range(C):
            row = np.zeros(C)
            row[i] = 1.0
            for j in range(i):
                row -= Lm[i, j] * Tm[j]
            Tm[i] = row
        u = Tm @ (b_c[:, None] * v_c)
        w = Tm @ ((b_c * np.exp(G))[:, None] * k_c)
        out.append(dict(q=q_c, k=k_c, G=G, Gam=Gam, L=Lm, T=Tm, u=u, w=w))
    return out, L_


def gdn_chunked(q, k, v, g, beta, h0, cu, scale, use_l2norm=True, chunk=64):
    """The page's chunked UT/WY evaluation (hyper-parallel
    ``_run_prepared_gdn_chunks``), each sequence chunked from its own start.
    Per chunk: v_new = u - w S;  o = (q o e^G) S + ((q k^T) o Gamma) v_new;
    S <- e^{G_C} S + (k o e^{G_C - G})^T v_new."""
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    qh, kh = _prep(q, k, scale, use_l2norm)
    N = len(cu) - 1
    o = np.zeros((T, Hv, dv))
    ht = np.zeros((N, Hv, dk, dv))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(Hv):
            a = h // grp
            S = np.zeros((dk, dv)) if h0 is None else h0[n, h].copy()
            chunks, L_ = _chunk_prepare(qh[s:e, a], kh[s:e, a], v[s:e, h], g[s:e, h], beta[s:e, h], chunk)
            outs = []
            for ch in chunks:
                v_new = ch["u"] - ch["w"] @ S
                attn = (ch["q"] @ ch["k"].T) * ch["Gam"]
                outs.append((ch["q"] * np.exp(ch["G"])[:, None]) @ S + attn @ v_new)
                GC = ch["G"][-1]
                S = np.exp(GC) * S + (ch["k"] * np.exp(GC - ch["G"])[:, None]).T @ v_new
            if outs:
                o[s:e, h] = np.concatenate(outs, axis=0)[:L_]
            ht[n, h] = S
    return o, ht


def gdn_state_summary(k, v, g, beta, cu, use_l2norm=True, chunk=64):
    """Affine summary of each sequence: S_out = M S_in + E
    (hyper-parallel ``_compute_gdn_state_summary_from_prepared``).  Per chunk
    M_c = e^{G_C} I - (k o e^{G_C - G})^T w and E_c = (k o e^{G_C - G})^T u,
    folded as E <- M_c E + E_c, M <- M_c M from E = 0, M = I.
    Returns M [N,Hv,dk,dk], E [N,Hv,dk,dv]."""
    T, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    kh = l2norm(k) if use_l2norm else k
    N = len(cu) - 1
    Ms = np.zeros((N, Hv, dk, dk))
    Es = np.zeros((N, Hv, dk, dv))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(Hv):
            a = h // grp
            chunks, _ = _chunk_prepare(kh[s:e, a], kh[s:e, a], v[s:e, h], g[s:e, h], beta[s:e, h], chunk)
            M = np.eye(dk)
            E = np.zeros((dk, dv))
            for ch in chunks:
                GC = ch["G"][-1]
                kd = ch["k"] * np.exp(GC - ch["G"])[:, None]
                Mc = np.exp(GC) * np.eye(dk) - kd.T @ ch["w"]
                Ec = kd.T @ ch["u"]
                E = Mc @ E + Ec
                M = Mc @ M
            Ms[n, h], Es[n, h] = M, E
    return Ms, Es


def merge_prefix_summaries(Ms, Es, rank):
    """hyper-parallel ``_merge_gdn_prefix_state_summaries_torch``: fold the
    summaries of shards 0..rank-1 from a zero state, h <- M_r h + E_r."""
    h = np.zeros_like(Es[0])
    for r in range(rank):
        h = Ms[r] @ h + Es[r]
    return h
