"""Seeded synthetic inputs shaped like diffusion-LM decoding steps.

This module only draws random numbers (torch RNG) and lays them out; it holds
none of the decision arithmetic.  Both the HIP path and the CPU oracle consume
the tensors it returns (the oracle through .cpu() copies).

Workloads (sizes from the decoding settings the pages describe: LLaDA / Dream
generations of 256 tokens in 32-token blocks, vocabularies of 126464 / 151936,
LLaDA's 32 layers x 32 heads with the last ~30% of layers averaged):

  tiny    1 x 32 rows,    V=4096,   fp32, sigma 1, every row planted, boost U(0,8),
          prev = cur + N(0, 0.3); one 32x32 attention map softmax(N(0,1)), fp32
  llada   1 x 256 rows,   V=126464, bf16, sigma 2, 60% planted, boost U(0,12),
          prev = cur + N(0, 0.5); (step extras: CAP on block 0 and a DAPD graph over
          the 256 rows with [1, 320, 768, 768] attention as in the dapd workload)
  dream   16 x 256 rows,  V=151936, bf16, sigma 2, every row planted, boost U(0,12), no prev
  dapd    8 x 256 rows,   V=126464, bf16, sigma 2, 60% planted, boost U(0,12), no prev;
          attention [8, 320, 768, 768] = softmax over keys of N(0, 1.5) logits, bf16;
          masked positions 512..767 (prompt 512 + generation 256)
  stress  64 x 1024 rows, V=126464, bf16, sigma 2, 50% planted, boost U(0,12),
          prev = cur + N(0, 0.5)

Planting (variant "peak"): a planted row's token is uniform over the vocabulary
and its logit is set to the row's background maximum plus U(0, boost).  Variant
"lit" adds U(0, boost) to the token's own logit instead.  Variant "cov" draws
planted tokens from a 16-id subset per sequence and puts, on 25% of rows, a
second peak (planted value minus U(4, 12)) at a neighbouring row's token, so
that argmax collisions and conflict scores near -16 occur.  For attention,
"cov" gives each masked position 3 random masked partners whose attention
logits get +4 in every map.

Every sequence b of a workload with seed s uses its own generator seeded
s * 1000 + b, so any subset of sequences can be regenerated alone.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    seed: int
    batch: int
    rows: int            # masked rows per sequence
    vocab: int
    dtype: torch.dtype
    sigma: float
    frac: float          # fraction of planted rows
    boost: float         # planted boost U(0, boost)
    prev_sigma: float | None
    # attention (DAPD-style) inputs
    n_lh: int = 0
    seq_len: int = 0     # S (prompt + generation)
    attn_sigma: float = 0.0
    attn_dtype: torch.dtype = torch.bfloat16

    @property
    def n_rows(self) -> int:
        return self.batch * self.rows


SPECS = {
    "tiny": Spec("tiny", 0, 1, 32, 4096, torch.float32, 1.0, 1.0, 8.0, 0.3,
                 n_lh=1, seq_len=32, attn_sigma=1.0, attn_dtype=torch.float32),
    "llada": Spec("llada", 1, 1, 256, 126464, torch.bfloat16, 2.0, 0.6, 12.0, 0.5,
                  n_lh=320, seq_len=768, attn_sigma=1.5),
    "dream": Spec("dream", 2, 16, 256, 151936, torch.bfloat16, 2.0, 1.0, 12.0, None),
    "dapd": Spec("dapd", 3, 8, 256, 126464, torch.bfloat16, 2.0, 0.6, 12.0, None,
                 n_lh=320, seq_len=768, attn_sigma=1.5),
    "stress": Spec("stress", 4, 64, 1024, 126464, torch.bfloat16, 2.0, 0.5, 12.0, 0.5),
}

# Decision-rule parameters per workload (page defaults unless the workload
# names others).
RULES = {
    "tiny": dict(tau=0.9, lam=1.0, l_min=4, l_max=32, tau_low=0.8, tau_high=0.95, gamma=-16.0,
                 k_max=32, dapd_tau=0.01, fast_block=(0, 32), cap_block=(0, 32)),
    "llada": dict(tau=0.9, lam=1.2, l_min=8, l_max=128, tau_low=0.8, tau_high=0.95,
                  gamma=-16.0, k_max=32, dapd_tau=0.01, fast_block=(0, 32), cap_block=(0, 32)),
    "dream": dict(tau_low=0.7, tau_high=0.95, gamma=-16.0, k_max=64),
    "dapd": dict(dapd_tau=0.01),
    "stress": dict(lam=1.2, l_min=8, l_max=128, tau_low=0.8, tau_high=0.95, gamma=-16.0,
                   k_max=128),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def seq_logits(spec: Spec, b: int, device, variant: str = "peak", rows: int | None = None,
               vocab: int | None = None):
    """fp32 (cur, prev) logits of sequence b: [rows, vocab] each (prev may be None)."""
    rows = spec.rows if rows is None else rows
    V = spec.vocab if vocab is None else vocab
    g = _gen(spec.seed * 1000 + b, device)
    x = torch.randn(rows, V, generator=g, device=device) * spec.sigma
    planted = torch.rand(rows, generator=g, device=device) < spec.frac
    if variant == "cov":
        ids = torch.randint(0, V, (16,), generator=g, device=device)
        tok = ids[torch.randint(0, 16, (rows,), generator=g, device=device)]
    else:
        tok = torch.randint(0, V, (rows,), generator=g, device=device)
    boost = torch.rand(rows, generator=g, device=device) * spec.boost
    r = torch.arange(rows, device=device)
    if variant == "lit":
        val = x[r, tok] + boost
    else:
        val = x.max(dim=1).values + boost
    x[r[planted], tok[planted]] = val[planted]
    if variant == "cov":
        second = (torch.rand(rows, generator=g, device=device) < 0.25) & planted
        nb = (r + 1) % rows
        drop = 4.0 + 8.0 * torch.rand(rows, generator=g, device=device)
        sel = r[second]
        x[sel, tok[nb[second]]] = val[second] - drop[second]
    prev = None
    if spec.prev_sigma is not None:
        prev = x + torch.randn(rows, V, generator=g, device=device) * spec.prev_sigma
    return x, prev


def logits(spec: Spec | str, device, variant: str = "peak", batch: int | None = None,
           rows: int | None = None, vocab: int | None = None):
    """Whole workload: cur [B*rows, V] in spec.dtype, prev (or None),
    seq_offsets int32 [B+1] and row_index int64 [B*rows] on `device`."""
    spec = SPECS[spec] if isinstance(spec, str) else spec
    B = spec.batch if batch is None else batch
    R = spec.rows if rows is None else rows
    V = spec.vocab if vocab is None else vocab
    cur = torch.empty(B * R, V, device=device, dtype=spec.dtype)
    prev = (torch.empty(B * R, V, device=device, dtype=spec.dtype)
            if spec.prev_sigma is not None else None)
    for b in range(B):
        x, p = seq_logits(spec, b, device, variant, rows=R, vocab=V)
        cur[b * R:(b + 1) * R] = x.to(spec.dtype)
        if prev is not None:
            prev[b * R:(b + 1) * R] = p.to(spec.dtype)
        del x, p
    seq_offsets = torch.arange(0, (B + 1) * R, R, device=device, dtype=torch.int32)
    row_index = torch.arange(B * R, device=device, dtype=torch.int64)
    return cur, prev, seq_offsets, row_index


def attention(spec: Spec | str, device, variant: str = "peak", batch: int | None = None,
              n_lh: int | None = None, seq_len: int | None = None,
              masked_pos: torch.Tensor | None = None):
    """Attention probabilities [B, n_lh, S, S] = softmax over keys of
    N(0, attn_sigma) logits, in spec.attn_dtype.  With variant "cov", each
    masked query gets 3 masked partners (+4 on those logits in every map)."""
    spec = SPECS[spec] if isinstance(spec, str) else spec
    B = spec.batch if batch is None else batch
    L = spec.n_lh if n_lh is None else n_lh
    S = spec.seq_len if seq_len is None else seq_len
    out = torch.empty(B, L, S, S, device=device, dtype=spec.attn_dtype)
    for b in range(B):
        g = _gen(spec.seed * 1000 + 500 + b, device)
        bias = None
        if variant == "cov" and masked_pos is not None:
            pos = masked_pos.to(device=device, dtype=torch.long)
            M = pos.numel()
            bias = torch.zeros(S, S, device=device)
            part = torch.randint(0, M, (M, 3), generator=g, device=device)
            bias[pos.unsqueeze(1).expand(M, 3), pos[part]] = 4.0
        for l0 in range(0, L, 32):
            l1 = min(L, l0 + 32)
            z = torch.randn(l1 - l0, S, S, generator=g, device=device) * spec.attn_sigma
            if bias is not None:
                z += bias
            out[b, l0:l1] = torch.softmax(z, dim=-1).to(spec.attn_dtype)
            del z
    return out


def gen_positions(spec: Spec | str, device, batch: int | None = None):
    """Masked positions of each sequence: the last `rows` positions of S
    (prompt first, then the generation), as int32 CSR with offsets."""
    spec = SPECS[spec] if isinstance(spec, str) else spec
    B = spec.batch if batch is None else batch
    S, M = spec.seq_len, spec.rows
    pos = torch.arange(S - M, S, device=device, dtype=torch.int32).repeat(B)
    offs = torch.arange(0, (B + 1) * M, M, device=device, dtype=torch.int32)
    return pos, offs
