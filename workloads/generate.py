"""Seeded generators for verify-step inputs.

Every tensor is drawn from its own torch.Generator, seeded from (seed, stream
name), so that changing one size does not perturb the other tensors.  The
sequence structure (KV lengths, draft lengths, page permutation) is always
drawn on the CPU, so it is the same whichever device the bulk data lands on.
Bulk data (Q/K/V, logits) is drawn on ``device``: the CPU and GPU random
streams differ, so a parity check must feed both sides the same generated
tensors (which is what the tests and the benchmark do).

Layouts (the ones the C ABI takes):
  q            bf16  [T_q, H_kv*G, d]      row q_start[b]+i is position i of seq b
  k_cache      bf16  [P, H_kv, page, d]    one (page, head) block is contiguous
  v_cache      bf16  [P, H_kv, page, d]    like K (spec.v_layout "key", the default), or
                     [P, H_kv, d, page]    each page stored d-major (V^T of its 16 keys; "dim")
  block_table  int32 [B, max_pages]        -1 past each sequence's last page
  kv_len       int32 [B]                   keys of seq b, including its 1+D_b block
  q_start      int32 [B+1]                 seq b owns rows q_start[b] .. q_start[b+1]-1
  target       fp32  [T_q, V]              target logits, one row per verify position
  draft        fp32  [T_d, V]              draft logits, row (q_start[b]-b)+i for i < D_b
  draft_tokens int32 [T_d]                 x_{i+1} drawn from draft row i
  uniforms     fp32  [T_q]                 u[q_start[b]+i]: test of draft i+1 (i < D_b);
                                           u[q_start[b]+D_b]: the sampling uniform
"""

from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence, Union

import torch

BF16_NAN_BITS = 0x7FC0


def _stream_seed(seed: int, name: str) -> int:
    h = hashlib.sha256(f"{seed}:{name}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, name: str, device: torch.device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_stream_seed(seed, name))
    return g


@dataclass
class WorkloadSpec:
    """Sizes and value distributions of one synthetic verify step.

    ``kv_len`` is an int (every sequence), a list (one per sequence) or
    ("lognormal", median, sigma, lo, hi).  ``draft_len`` is an int (every
    sequence), a list (one per sequence) or a tuple of choices drawn uniformly
    per sequence.  ``alpha`` switches the draft distribution to the
    fixed-acceptance-rate construction q = (1-lam) p + lam/V (see generate()).
    """

    name: str
    batch: int
    kv_heads: int
    group: int
    head_dim: int
    kv_len: Union[int, tuple]
    draft_len: Union[int, tuple]
    vocab: int
    mode: str = "stochastic"           # or "greedy"
    page_size: int = 16
    target_std: float = 3.0
    draft_noise_std: float = 1.0
    alpha: Optional[float] = None
    draft_pick: str = "sample"         # "sample" from q, or "argmax" of the draft logits
    extra_pool_pages: int = 0          # unused pages mixed into the shared pool
    v_layout: str = "key"              # V pages key-major like K ("key") or d-major ("dim")
    seed: int = 0

    def with_(self, **kw) -> "WorkloadSpec":
        return replace(self, **kw)

    @property
    def query_heads(self) -> int:
        return self.kv_heads * self.group

    def max_draft(self) -> int:
        return self.draft_len if isinstance(self.draft_len, int) else max(self.draft_len)


@dataclass
class VerifyInputs:
    spec: WorkloadSpec
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    kv_len: torch.Tensor
    q_start: torch.Tensor
    target_logits: torch.Tensor
    draft_logits: Optional[torch.Tensor]
    draft_tokens: torch.Tensor
    uniforms: torch.Tensor
    max_draft: int
    extras: dict = field(default_factory=dict)

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def group(self) -> int:
        return self.spec.group

    def to(self, device) -> "VerifyInputs":
        def mv(t):
            return None if t is None else t.to(device)
        return replace(
            self,
            q=mv(self.q), k_cache=mv(self.k_cache), v_cache=mv(self.v_cache),
            block_table=mv(self.block_table), kv_len=mv(self.kv_len), q_start=mv(self.q_start),
            target_logits=mv(self.target_logits), draft_logits=mv(self.draft_logits),
            draft_tokens=mv(self.draft_tokens), uniforms=mv(self.uniforms),
        )


def _structure(spec: WorkloadSpec):
    """KV lengths, draft lengths and the page assignment, drawn on the CPU."""
    B = spec.batch
    if isinstance(spec.kv_len, int):
        kv = torch.full((B,), spec.kv_len, dtype=torch.int64)
    elif isinstance(spec.kv_len, list):
        kv = torch.tensor(spec.kv_len, dtype=torch.int64)
        assert len(kv) == B
    else:
        kind, median, sigma, lo, hi = spec.kv_len
        assert kind == "lognormal"
        z = torch.randn(B, generator=_gen(spec.seed, "kv_len", torch.device("cpu")), dtype=torch.float64)
        kv = torch.exp(math.log(median) + sigma * z).round().clamp(lo, hi).to(torch.int64)
    if isinstance(spec.draft_len, int):
        dl = torch.full((B,), spec.draft_len, dtype=torch.int64)
    elif isinstance(spec.draft_len, list):
        dl = torch.tensor(spec.draft_len, dtype=torch.int64)
        assert len(dl) == B
    else:
        choices = torch.tensor(list(spec.draft_len), dtype=torch.int64)
        idx = torch.randint(len(choices), (B,), generator=_gen(spec.seed, "draft_len", torch.device("cpu")))
        dl = choices[idx]
    ps = spec.page_size
    pages = (kv + ps - 1) // ps
    max_pages = int(pages.max()) if B > 0 else 1
    pool = int(pages.sum()) + spec.extra_pool_pages
    perm = torch.randperm(max(pool, 1), generator=_gen(spec.seed, "pages", torch.device("cpu")))
    bt = torch.full((B, max(max_pages, 1)), -1, dtype=torch.int64)
    off = 0
    for b in range(B):
        n = int(pages[b])
        bt[b, :n] = perm[off:off + n]
        off += n
    q_start = torch.zeros(B + 1, dtype=torch.int64)
    q_start[1:] = torch.cumsum(dl + 1, 0)
    return kv, dl, bt, q_start, max(pool, 1)


def draft_pool_pages(spec: WorkloadSpec) -> int:
    return _structure(spec)[4]


def _randn_bf16(shape, gen, device, chunk_rows=4096):
    """N(0,1) drawn in fp32 and rounded to bf16 (round-to-nearest-even)."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        flat[r0:r1] = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                                  dtype=torch.float32).to(torch.bfloat16)
    return out


def _gumbel_argmax(logits64: torch.Tensor, gen, device) -> torch.Tensor:
    """One token per row distributed as softmax(logits) (Gumbel-max trick)."""
    u = torch.rand(logits64.shape, generator=gen, device=device, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    return torch.argmax(logits64 - torch.log(-torch.log(u)), dim=-1)


def generate(spec: WorkloadSpec, device="cpu", poison_tail: bool = False) -> VerifyInputs:
    """Draw one verify step's inputs.

    poison_tail writes bf16 NaN into the unused slots of each sequence's last
    page (keys at or past kv_len), which a correct kernel never reads into a
    result.
    """
    device = torch.device(device)
    kv, dl, bt, q_start, pool = _structure(spec)
    B, Hkv, G, d, ps, V = spec.batch, spec.kv_heads, spec.group, spec.head_dim, spec.page_size, spec.vocab
    Hq = Hkv * G
    T_q = int(q_start[-1]) if B > 0 else 0
    T_d = T_q - B

    q = _randn_bf16((max(T_q, 0), Hq, d), _gen(spec.seed, "q", device), device)
    k_cache = _randn_bf16((pool, Hkv, ps, d), _gen(spec.seed, "k", device), device)
    # values are drawn key-major; "dim" stores each page transposed (the logical V is the same draw)
    if spec.v_layout not in ("key", "dim"):
        raise ValueError(f"v_layout {spec.v_layout!r}: 'key' or 'dim'")
    v_cache = _randn_bf16((pool, Hkv, ps, d), _gen(spec.seed, "v", device), device)
    if spec.v_layout == "dim":
        v_cache = v_cache.transpose(2, 3).contiguous()
    if poison_tail:
        kb = k_cache.view(torch.int16)
        vb = v_cache.view(torch.int16)
        for b in range(B):
            n = int(kv[b])
            if n % ps:
                page = int(bt[b, (n - 1) // ps])
                kb[page, :, n % ps:, :] = BF16_NAN_BITS
                if spec.v_layout == "dim":
                    vb[page, :, :, n % ps:] = BF16_NAN_BITS
                else:
                    vb[page, :, n % ps:, :] = BF16_NAN_BITS

    target = torch.randn((T_q, V), generator=_gen(spec.seed, "target", device), device=device,
                         dtype=torch.float32) * spec.target_std
    # draft row (q_start[b]-b)+i pairs with target row q_start[b]+i, i < D_b
    trow = torch.cat([torch.arange(int(q_start[b]), int(q_start[b]) + int(dl[b])) for b in range(B)]) \
        if T_d > 0 else torch.zeros(0, dtype=torch.int64)
    trow_dev = trow.to(device)
    extras = {"draft_len": dl, "kv_len": kv, "pool_pages": pool}
    if spec.alpha is not None:
        # Synthetic fixed acceptance rate: q = (1-lam) p + lam/V with
        # lam = (1-alpha)/TV(p, uniform), so sum_x min(p, q) = alpha exactly.
        # p is needed here to build the synthetic drafter's q, not by the verify step.
        p = torch.softmax(target[trow_dev].double(), dim=-1)
        tv = 0.5 * (p - 1.0 / V).abs().sum(-1, keepdim=True)
        lam = (1.0 - spec.alpha) / tv
        if T_d and float(lam.max()) > 1.0:
            raise ValueError(f"alpha={spec.alpha} unreachable: need TV >= {1 - spec.alpha}")
        qd = (1.0 - lam) * p + lam / V
        draft64 = torch.log(qd)
        extras["lambda"] = lam.squeeze(-1).cpu()
    else:
        noise = torch.randn((T_d, V), generator=_gen(spec.seed, "draft_noise", device), device=device,
                            dtype=torch.float32) * spec.draft_noise_std
        draft64 = (target[trow_dev] + noise).double() if T_d else torch.zeros((0, V), dtype=torch.float64,
                                                                               device=device)
    draft = draft64.to(torch.float32)
    if spec.draft_pick == "argmax":
        tokens = torch.argmax(draft, dim=-1) if T_d else torch.zeros(0, dtype=torch.int64, device=device)
    else:
        tokens = _gumbel_argmax(draft.double(), _gen(spec.seed, "draft_pick", device), device) if T_d \
            else torch.zeros(0, dtype=torch.int64, device=device)
    uniforms = torch.rand((T_q,), generator=_gen(spec.seed, "uniforms", device), device=device,
                          dtype=torch.float32)

    return VerifyInputs(
        spec=spec,
        q=q,
        k_cache=k_cache,
        v_cache=v_cache,
        block_table=bt.to(torch.int32).to(device),
        kv_len=kv.to(torch.int32).to(device),
        q_start=q_start.to(torch.int32).to(device),
        target_logits=target,
        draft_logits=draft if spec.mode == "stochastic" else None,
        draft_tokens=tokens.to(torch.int32),
        uniforms=uniforms,
        max_draft=spec.max_draft(),
        extras=extras,
    )
