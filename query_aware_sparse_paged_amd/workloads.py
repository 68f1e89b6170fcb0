"""Seeded synthetic decode workloads.

This module only draws inputs: a KV pool with pages scattered at a seeded
permutation, a page table, sequence lengths, the decode query and the new
token.  It holds none of the method's arithmetic (no summaries, scores,
selection or attention), so the GPU library and the CPU oracle can both be fed
from it.

Workloads (shapes of the long-context agent / decode settings the method
targets; the SparseEngine article, blog.ontle.kr/blog/332, names Llama-3.1-8B
as an evaluation model and GLM-4.7-Flash as the MLA model):

  tiny_b1_4k        batch 1, 32 q / 8 KV heads, d 128, 4096 tokens, page 16,
                    256 pages in a 512-page pool; keep 1 sink + 4 local +
                    top-32.
  llama8b_b32_32k   batch 32, 32 q / 8 KV heads, d 128, 32768 tokens, page 16;
                    keys N(0,1) times a per-(KV head, channel) LogNormal(0,0.5)
                    scale; 1 sink + 8 local + top-119 (2048-token budget).
  needle_b8_128k    batch 8, 131072 tokens, page 16; 64 needle keys per
                    sequence pointing along the group's mean query direction;
                    1 sink + 8 local + top-247 (4096-token budget).
  ragged_b64_mixed  64 sequences, lengths uniform in [4096, 65536]; KV heads
                    0-3 static A-shape (4 sink tokens + 1024-token window),
                    KV heads 4-7 query-aware 1 + 8 + top-55 (1024 tokens).
  mla_b16_64k       batch 16, 128 q heads over one latent KV head of 576
                    channels (values = first 512), 65536 tokens, page 64,
                    scale 1/sqrt(192); 1 sink + 2 local + top-29 (2048 tokens).

Values are drawn in fp32 from torch's seeded generator on the requested device
and rounded to bf16 (round to nearest even).  The same seed gives the same
inputs on the same device type; CPU and GPU streams differ.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass
class Spec:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_k: int
    head_dim_v: int
    page_size: int
    seq_len: int                      # fixed length, or the upper end of a range
    seq_len_min: Optional[int] = None  # set: lengths uniform in [seq_len_min, seq_len]
    pool_pages: Optional[int] = None   # None: twice the pages in use
    n_sink_pages: int = 1
    n_local_pages: int = 8
    top_k: int = 119
    sink_tokens: int = 0
    window_tokens: int = 0
    static_heads: Optional[List[int]] = None
    scale: Optional[float] = None      # None: 1/sqrt(head_dim_k)
    v_from_k: bool = False
    key_channel_lognormal_sigma: float = 0.0
    needles: int = 0
    seed: int = 0


SPECS = {
    "tiny_b1_4k": Spec("tiny_b1_4k", 1, 32, 8, 128, 128, 16, 4096, pool_pages=512,
                       n_sink_pages=1, n_local_pages=4, top_k=32, seed=1),
    "llama8b_b32_32k": Spec("llama8b_b32_32k", 32, 32, 8, 128, 128, 16, 32768,
                            n_sink_pages=1, n_local_pages=8, top_k=119,
                            key_channel_lognormal_sigma=0.5, seed=2),
    "needle_b8_128k": Spec("needle_b8_128k", 8, 32, 8, 128, 128, 16, 131072,
                           n_sink_pages=1, n_local_pages=8, top_k=247, needles=64, seed=3),
    "ragged_b64_mixed": Spec("ragged_b64_mixed", 64, 32, 8, 128, 128, 16, 65536, seq_len_min=4096,
                             n_sink_pages=1, n_local_pages=8, top_k=55, sink_tokens=4,
                             window_tokens=1024, static_heads=[1, 1, 1, 1, 0, 0, 0, 0], seed=4),
    "mla_b16_64k": Spec("mla_b16_64k", 16, 128, 1, 576, 512, 64, 65536,
                        n_sink_pages=1, n_local_pages=2, top_k=29, scale=1.0 / math.sqrt(192.0),
                        v_from_k=True, seed=5),
}


@dataclass
class Workload:
    spec: Spec
    seq_lens: torch.Tensor        # int32 [B], current token included
    page_table: torch.Tensor      # int32 [B][stride]; entry P_b is a spare page for one append
    q: torch.Tensor               # bf16 [B][Hq][Dk]
    k_pool: torch.Tensor          # bf16 [pool][Hkv][ps][Dk]
    v_pool: Optional[torch.Tensor]  # bf16 [pool][Hkv][Dv][ps], None for latent KV
    k_new: torch.Tensor           # bf16 [B][Hkv][Dk]: the key stored at position L-1
    v_new: Optional[torch.Tensor]  # bf16 [B][Hkv][Dv]: the value stored at position L-1
    needle_pos: Optional[torch.Tensor] = None  # int64 [B][needles]
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        s = self.spec.scale
        return float(s) if s is not None else 1.0 / math.sqrt(self.spec.head_dim_k)

    @property
    def num_pool_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def _randn_bf16(shape, gen, device, chunk_rows=4096):
    """N(0,1) drawn in fp32, rounded to bf16, generated in row chunks."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def make(name: str, seed: Optional[int] = None, device="cpu", batch: Optional[int] = None,
         seq_len: Optional[int] = None, seq_len_min: Optional[int] = None,
         **overrides) -> Workload:
    """Draws workload `name`.  batch / seq_len / seq_len_min / spec fields may be
    overridden to get smaller cases of the same recipe."""
    base = SPECS[name]
    spec = Spec(**{**base.__dict__, **overrides})
    if batch is not None:
        spec.batch = batch
    if seq_len is not None:
        spec.seq_len = seq_len
        if seq_len_min is None and spec.seq_len_min is not None:
            spec.seq_len_min = max(1, min(spec.seq_len_min, seq_len))
    if seq_len_min is not None:
        spec.seq_len_min = seq_len_min
    if seed is None:
        seed = spec.seed
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))

    B, Hq, Hkv, Dk, Dv, ps = (spec.batch, spec.num_q_heads, spec.num_kv_heads,
                              spec.head_dim_k, spec.head_dim_v, spec.page_size)
    # sequence lengths
    if spec.seq_len_min is not None:
        seq_lens = torch.randint(spec.seq_len_min, spec.seq_len + 1, (B,), generator=gen,
                                 device=device).to(torch.int32)
    else:
        seq_lens = torch.full((B,), spec.seq_len, dtype=torch.int32, device=device)
    lens = seq_lens.cpu().tolist()
    pages = [(L + ps - 1) // ps for L in lens]
    used = sum(pages)
    stride = max(pages + [0]) + 1                  # one spare page per sequence
    pool = spec.pool_pages if spec.pool_pages is not None else 2 * max(used, 1)
    pool = max(pool, used + B)

    # physical placement: the first `used` entries of a seeded permutation,
    # then one spare page per sequence
    perm = torch.randperm(pool, generator=gen, device=device).to(torch.int32)
    page_table = torch.full((B, stride), -1, dtype=torch.int32, device=device)
    off = 0
    for b in range(B):
        page_table[b, :pages[b]] = perm[off:off + pages[b]]
        off += pages[b]
    for b in range(B):
        page_table[b, pages[b]] = perm[used + b]
    used_phys = perm[:used].long()

    # pools: unused pages are zero
    k_pool = torch.zeros((pool, Hkv, ps, Dk), dtype=torch.bfloat16, device=device)
    k_used = _randn_bf16((used, Hkv, ps, Dk), gen, device)
    if spec.key_channel_lognormal_sigma > 0:
        ch = torch.exp(spec.key_channel_lognormal_sigma *
                       torch.randn((Hkv, Dk), generator=gen, device=device, dtype=torch.float32))
        for r0 in range(0, used, 4096):
            r1 = min(used, r0 + 4096)
            k_used[r0:r1] = (k_used[r0:r1].float() * ch[None, :, None, :]).to(torch.bfloat16)
    k_pool[used_phys] = k_used
    del k_used
    v_pool = None
    if not spec.v_from_k:
        v_pool = torch.zeros((pool, Hkv, Dv, ps), dtype=torch.bfloat16, device=device)
        v_pool[used_phys] = _randn_bf16((used, Hkv, Dv, ps), gen, device)

    q = torch.randn((B, Hq, Dk), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)

    # needles: keys along the group's mean query direction, at the norm of a
    # typical N(0,1) key (4 * sqrt(Dk)), written at seeded positions inside the
    # scored page range [n_sink*ps, L - n_local*ps)
    needle_pos = None
    if spec.needles > 0:
        G = Hq // Hkv
        direction = q.float().view(B, Hkv, G, Dk).mean(dim=2)
        direction = direction / direction.norm(dim=-1, keepdim=True)
        needle = (4.0 * math.sqrt(Dk) * direction).to(torch.bfloat16)    # [B][Hkv][Dk]
        needle_pos = torch.empty((B, spec.needles), dtype=torch.int64, device=device)
        for b in range(B):
            lo_t = spec.n_sink_pages * ps
            hi_t = lens[b] - spec.n_local_pages * ps
            span = hi_t - lo_t
            assert span >= spec.needles, "sequence too short for the needles"
            pos = lo_t + torch.randperm(span, generator=gen, device=device)[:spec.needles]
            needle_pos[b] = pos
            phys = page_table[b].long()[pos // ps]
            slot = pos % ps
            for g in range(Hkv):
                k_pool[phys, g, slot, :] = needle[b, g][None, :].expand(spec.needles, Dk)

    # the token at position L-1, as an append would write it
    last = torch.tensor([L - 1 for L in lens], dtype=torch.int64, device=device)
    bidx = torch.arange(B, device=device)
    phys_last = page_table[bidx, (last // ps)].long() if B > 0 else last
    slot_last = last % ps
    k_new = k_pool[phys_last, :, slot_last, :].clone() if B > 0 else \
        torch.zeros((0, Hkv, Dk), dtype=torch.bfloat16, device=device)
    v_new = None
    if v_pool is not None:
        v_new = v_pool[phys_last, :, :, slot_last].clone() if B > 0 else \
            torch.zeros((0, Hkv, Dv), dtype=torch.bfloat16, device=device)
    return Workload(spec, seq_lens, page_table, q, k_pool, v_pool, k_new, v_new, needle_pos)


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def from_bits(a, device="cpu") -> torch.Tensor:
    """numpy uint16 bit patterns -> bf16 tensor."""
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def drafts(w: Workload, n: int, seed: int, device="cpu"):
    """Draft tokens of a multi-query step over workload w: queries
    [B][n][Hq][Dk], keys [B][n][Hkv][Dk] and values [B][n][Hkv][Dv] (None
    when values are key channels), N(0,1) in fp32 rounded to bf16, from a
    CPU generator seeded with `seed`."""
    s = w.spec
    gen = torch.Generator().manual_seed(int(seed))
    B = int(w.seq_lens.shape[0])
    q = _randn_bf16((B, n, s.num_q_heads, s.head_dim_k), gen, "cpu").to(device)
    k = _randn_bf16((B, n, s.num_kv_heads, s.head_dim_k), gen, "cpu").to(device)
    v = None if s.v_from_k else _randn_bf16((B, n, s.num_kv_heads, s.head_dim_v), gen, "cpu").to(device)
    return q, k, v
