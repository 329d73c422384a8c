"""Seeded synthetic inputs for block-sparse landmark attention.

This module only draws random tensors; it holds none of the method's arithmetic.  It is the
one module shared by the device path's tests/benchmark and the float64 oracle's tests.

Recipes (the design notes list them with their sources):

* ``iid``: q, k, v ~ N(0, 1).
* ``clustered``: for every (sequence, kv head) there are ``n_centres`` unit centres
  C = normalise(N(0, I_D)).  Each 64-token key block j draws one centre z_j uniformly and its
  keys are k_t = 3 C[z_j] + N(0, I).  Each query block c >= 1 is aimed at earlier blocks: when
  c > n_aim, n_aim blocks are drawn uniformly from 0..c-1 (with replacement) and shared by all
  heads of the kv group; every (head, token) picks one of those n_aim slots uniformly; when
  1 <= c <= n_aim every (head, token) picks an earlier block uniformly from 0..c-1.  The query
  is q = 3 C[z_target] + N(0, I).  Query block 0 is pure noise.  v ~ N(0, 1).
* decode: the same keys; the one query token of each sequence is aimed at n_aim blocks drawn
  from 0..c-1 (c = the block of the last token); each query head picks one slot.

Every tensor has its own generator stream, seeded with seed * 1000 + tensor_id, so changing
one tensor's shape leaves the others unchanged.  Values are drawn in float32 and cast to the
working dtype (round-to-nearest-even) at the end.
"""

from __future__ import annotations

import torch

BLOCK = 64

# The five workloads: the tiny fp32 check, GQA prefill at 32K, SAS prefill at 128K (headline),
# batched decode over 128K caches (headline) and HiLS prefill at 1M tokens.
WORKLOADS = {
    "tiny_f32_4k": dict(kind="prefill", B=1, Hq=1, Hkv=1, D=64, T=4096, dtype="f32", topk=8,
                        mode="plain", data="iid"),
    "gqa_bf16_32k": dict(kind="prefill", B=1, Hq=32, Hkv=8, D=128, T=32768, dtype="bf16",
                         topk=16, mode="plain", data="clustered", n_centres=256, n_aim=16),
    "sas_bf16_128k": dict(kind="prefill", B=1, Hq=32, Hkv=8, D=128, T=131072, dtype="bf16",
                          topk=32, mode="sas", data="clustered", n_centres=256, n_aim=16),
    "decode_bf16_32x128k": dict(kind="decode", B=32, Hq=64, Hkv=8, D=128, T=131072,
                                dtype="bf16", topk=64, mode="plain", data="clustered",
                                n_centres=256, n_aim=16),
    "hils_bf16_1m": dict(kind="prefill", B=1, Hq=32, Hkv=8, D=128, T=1048576, dtype="bf16",
                         topk=32, mode="hils", data="clustered", n_centres=4096, n_aim=16),
    # ragged serving batch: 32 sequences of 16K..128K tokens in shuffled 64-token pages
    "decode_paged_bf16_32x16k_128k": dict(kind="decode_paged", B=32, Hq=64, Hkv=8, D=128,
                                          T_min=16384, T=131072, dtype="bf16", topk=64,
                                          mode="plain", data="clustered", n_centres=256,
                                          n_aim=16),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tensor_id)
    return g


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _centres(B, Hkv, n_centres, D, gen, device):
    C = _randn((B, Hkv, n_centres, D), gen, device)
    return C / C.norm(dim=-1, keepdim=True)


def make_prefill(B, Hq, Hkv, T, D, dtype="bf16", data="iid", seed=0, device="cpu",
                 n_centres=256, n_aim=16, block=BLOCK):
    """q [B,Hq,T,D], k/v [B,Hkv,T,D] in the working dtype, contiguous, on `device`."""
    tdt = TORCH_DTYPE[dtype]
    G = Hq // Hkv
    NB = (T + block - 1) // block
    v = _randn((B, Hkv, T, D), _gen(device, seed, 3), device).to(tdt)
    if data == "iid":
        q = _randn((B, Hq, T, D), _gen(device, seed, 1), device).to(tdt)
        k = _randn((B, Hkv, T, D), _gen(device, seed, 2), device).to(tdt)
        return q, k, v
    if data != "clustered":
        raise ValueError(f"unknown data recipe {data!r}")
    gc = _gen(device, seed, 4)
    C = _centres(B, Hkv, n_centres, D, gc, device)                           # [B,Hkv,n,D]
    z = torch.randint(0, n_centres, (B, Hkv, NB), generator=gc, device=device)
    blk_of_t = torch.arange(T, device=device) // block                        # [T]
    k = torch.empty((B, Hkv, T, D), dtype=tdt, device=device)
    gk = _gen(device, seed, 2)
    for b in range(B):
        for g in range(Hkv):
            cent = C[b, g][z[b, g][blk_of_t]]                                 # [T,D]
            k[b, g] = (3.0 * cent + _randn((T, D), gk, device)).to(tdt)
    # aimed sets: [B,Hkv,NB,n_aim], block indices in [0, c) for c >= 1
    ga = _gen(device, seed, 5)
    cvec = torch.arange(NB, device=device, dtype=torch.float32)
    u = torch.rand((B, Hkv, NB, n_aim), generator=ga, device=device)
    aim = torch.floor(u * cvec[None, None, :, None]).long()
    q = torch.empty((B, Hq, T, D), dtype=tdt, device=device)
    gq = _gen(device, seed, 1)
    cblk = blk_of_t                                                            # [T]
    for b in range(B):
        for h in range(Hq):
            g = h // G
            slot = torch.randint(0, n_aim, (T,), generator=gq, device=device)
            u2 = torch.rand((T,), generator=gq, device=device)
            direct = torch.floor(u2 * cblk.float()).long()                     # in [0, c)
            via_aim = aim[b, g][cblk, slot]
            target = torch.where(cblk > n_aim, via_aim, direct)
            cent = C[b, g][z[b, g][target]]                                    # [T,D]
            cent = torch.where((cblk == 0)[:, None], torch.zeros_like(cent), cent)
            q[b, h] = (3.0 * cent + _randn((T, D), gq, device)).to(tdt)
    return q, k, v


def make_decode(B, Hq, Hkv, Tk, D, dtype="bf16", data="clustered", seed=0, device="cpu",
                n_centres=256, n_aim=16, block=BLOCK):
    """q [B,Hq,D] (the query at position Tk-1), kc/vc [B,Hkv,Tk,D] (the cache)."""
    tdt = TORCH_DTYPE[dtype]
    G = Hq // Hkv
    NB = (Tk + block - 1) // block
    vc = _randn((B, Hkv, Tk, D), _gen(device, seed, 3), device).to(tdt)
    if data == "iid":
        q = _randn((B, Hq, D), _gen(device, seed, 1), device).to(tdt)
        kc = _randn((B, Hkv, Tk, D), _gen(device, seed, 2), device).to(tdt)
        return q, kc, vc
    gc = _gen(device, seed, 4)
    C = _centres(B, Hkv, n_centres, D, gc, device)
    z = torch.randint(0, n_centres, (B, Hkv, NB), generator=gc, device=device)
    blk_of_t = torch.arange(Tk, device=device) // block
    kc = torch.empty((B, Hkv, Tk, D), dtype=tdt, device=device)
    gk = _gen(device, seed, 2)
    for b in range(B):
        for g in range(Hkv):
            cent = C[b, g][z[b, g][blk_of_t]]
            kc[b, g] = (3.0 * cent + _randn((Tk, D), gk, device)).to(tdt)
    c = (Tk - 1) // block
    ga = _gen(device, seed, 5)
    gq = _gen(device, seed, 1)
    if c == 0:
        q = _randn((B, Hq, D), gq, device).to(tdt)
        return q, kc, vc
    aim = torch.floor(torch.rand((B, Hkv, n_aim), generator=ga, device=device) * c).long()
    slot = torch.randint(0, n_aim, (B, Hq), generator=gq, device=device)
    hg = torch.arange(Hq, device=device) // G
    bidx = torch.arange(B, device=device)[:, None].expand(B, Hq)
    gidx = hg[None, :].expand(B, Hq)
    target = aim[bidx, gidx, slot]                                             # [B,Hq]
    cent = C[bidx, gidx, z[bidx, gidx, target]]                                # [B,Hq,D]
    q = (3.0 * cent + _randn((B, Hq, D), gq, device)).to(tdt)
    return q, kc, vc


def make_paged_decode(lens, Hq, Hkv, D, dtype="bf16", data="clustered", seed=0, device="cpu",
                      n_centres=256, n_aim=16, spare_pages=16, block=BLOCK):
    """A ragged decode batch in a paged cache.

    Sequence b (len lens[b]) is make_decode's cache for one sequence (seed + b); its blocks are
    scattered over a pool of 64-token pages [n_pages,Hkv,64,D] in a seeded random order, with
    `spare_pages` unused pages.  Returns q [B,Hq,D], k_pool, v_pool, page_table [B,NB] int32
    (NB = the longest sequence's blocks; unused entries point at page 0) and seq_lens [B] int32.
    """
    B = len(lens)
    nblk = [(int(L) + block - 1) // block for L in lens]
    NB = max(nblk)
    n_pages = sum(nblk) + spare_pages
    tdt = TORCH_DTYPE[dtype]
    k_pool = torch.zeros((n_pages, Hkv, block, D), dtype=tdt, device=device)
    v_pool = torch.zeros((n_pages, Hkv, block, D), dtype=tdt, device=device)
    order = torch.randperm(n_pages, generator=_gen("cpu", seed, 9)).to(device)
    table = torch.zeros((B, NB), dtype=torch.int32, device=device)
    qs = []
    nxt = 0
    for b, L in enumerate(lens):
        L = int(L)
        q, kc, vc = make_decode(1, Hq, Hkv, L, D, dtype, data, seed=seed + b, device=device,
                                n_centres=n_centres, n_aim=n_aim, block=block)
        qs.append(q)
        pages = order[nxt:nxt + nblk[b]]
        nxt += nblk[b]
        pad = nblk[b] * block - L
        for src, pool in ((kc, k_pool), (vc, v_pool)):
            t = torch.nn.functional.pad(src[0], (0, 0, 0, pad))            # [Hkv, nblk*64, D]
            pool[pages] = t.view(Hkv, nblk[b], block, D).permute(1, 0, 2, 3)
        table[b, : nblk[b]] = pages.to(torch.int32)
        del kc, vc
    seq_lens = torch.tensor([int(L) for L in lens], dtype=torch.int32, device=device)
    return torch.cat(qs, 0), k_pool, v_pool, table, seq_lens

