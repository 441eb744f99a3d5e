"""Seeded synthetic decode-step and chunk inputs.

This module only draws inputs; it holds none of the method's arithmetic (no
slot mapping, append, gather, softmax or fp8 rounding of its own).  Both the
HIP path and the CPU oracle consume what it returns.

Shapes and distributions follow the decode workloads this library is
measured on:

* ``tiny``      -- fp32, B=3, contexts {5, 17, 33} before the append,
  H_Q=4, H_KV=2, d_h=8, 4-slot blocks, a 32-block pool;
* ``llama8b``   -- one Llama-3.1-8B-style layer: bf16, B=32, H_Q=32, H_KV=8,
  d_h=128, 16-slot blocks, contexts uniform in [512, 4096] before the append;
* ``long32k``   -- same heads, B=8, every context 32,768 after the append
  (2,048 blocks per request);
* ``shared_prefix`` -- B=64, every table maps the same 75 blocks (a
  1,200-token prefix, page 3 "xf_kv_cache", "End-to-end flow"), then 600
  private prompt tokens plus a decode offset uniform in [0, 900]; 32 layers,
  each with its own pools and inputs, one shared block table;
* ``fp8_mqa`` / ``fp8_gqa`` / ``fp8_mha`` -- B=128, H_Q=32, H_KV=1 / 8 / 32,
  fp8 E4M3 K/V with one fp32 scale per (physical block, KV head), bf16 Q,
  contexts clip(round(2048 * e^Z), 128, 16384) with Z ~ N(0, 1);
* ``tiny_chunks`` -- the ``tiny`` shapes with a chunk of new tokens: request
  0 processes tokens 4..7 of a 12-token prompt taken in chunks of four
  (page 1, section 21.3), requests 1 and 2 decode one token each (contexts
  18 and 34 after the step);
* ``prefix_hit`` -- B=64 requests whose tables map the same 75 blocks (a
  1,200-token prefix) and then process their 600 unshared prompt tokens as
  one chunk (page 3, "End-to-end flow"): 38,400 new tokens, each attending
  to the shared prefix and to the chunk up to itself; Llama-3.1-8B-style
  heads, bf16, one layer.

Request b brings n_b new tokens (one for a decode step); ``query_start`` is
their prefix sum ([B + 1], starting at 0), and new K, V and Q rows are laid
out [sum n_b, heads, d_h] in request order.  For decode workloads this is
[B, heads, d_h], so their draws are the same as with one token per request.

Recipe (fixed order of draws from one seeded ``torch.Generator``):
context lengths -> physical-id permutation -> K pool -> V pool -> new K ->
new V -> Q.  Every pool slot, used or not, holds an N(0, 1) draw rounded
(RNE) to the storage type, so unused slots hold finite garbage.  Physical
ids: the pool has ceil(1.25 * blocks needed) blocks (32 for ``tiny``); a
random permutation of all ids is dealt out in table order (request 0's
blocks first), and table entries past a request's last block are -1.
For fp8 pools the generator draws fp32 values and picks
scale[p, h] = max(amax of the block's drawn values for head h, amax of the
new K (or V) values of head h over the batch, 2**-120) / 448, so that no
appended value overflows; the stored codes are torch's own float32 ->
float8_e4m3fn conversion of value / scale (a library routine).

Context lengths are reported *after* the append (the query reads its own new
key, page 1 "KV cache: Generation state, latency, and allocation", section
21.1), so every drawn "before" length gets +1, except ``long32k`` whose
32,768 is the length after the append.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPE_BYTES = {"f32": 4, "bf16": 2, "fp8_e4m3": 1}
_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16,
                "fp8_e4m3": torch.float8_e4m3fn}

CONFIGS = {
    "tiny": dict(B=3, H_Q=4, H_KV=2, d_h=8, block_size=4, kv_dtype="f32",
                 q_dtype="f32", layers=1, seed=0, lens="fixed",
                 lens_before=(5, 17, 33), pool_blocks=32),
    "llama8b": dict(B=32, H_Q=32, H_KV=8, d_h=128, block_size=16, kv_dtype="bf16",
                    q_dtype="bf16", layers=1, seed=1, lens="uniform", lo=512, hi=4096),
    "long32k": dict(B=8, H_Q=32, H_KV=8, d_h=128, block_size=16, kv_dtype="bf16",
                    q_dtype="bf16", layers=1, seed=2, lens="const_after", n_after=32768),
    "shared_prefix": dict(B=64, H_Q=32, H_KV=8, d_h=128, block_size=16, kv_dtype="bf16",
                          q_dtype="bf16", layers=32, seed=3, lens="shared",
                          shared_tokens=1200, private_tokens=600, offset_hi=900),
    "fp8_mqa": dict(B=128, H_Q=32, H_KV=1, d_h=128, block_size=16, kv_dtype="fp8_e4m3",
                    q_dtype="bf16", layers=1, seed=4, lens="lognormal", median=2048,
                    lo=128, hi=16384),
    "fp8_gqa": dict(B=128, H_Q=32, H_KV=8, d_h=128, block_size=16, kv_dtype="fp8_e4m3",
                    q_dtype="bf16", layers=1, seed=4, lens="lognormal", median=2048,
                    lo=128, hi=16384),
    "fp8_mha": dict(B=128, H_Q=32, H_KV=32, d_h=128, block_size=16, kv_dtype="fp8_e4m3",
                    q_dtype="bf16", layers=1, seed=4, lens="lognormal", median=2048,
                    lo=128, hi=16384),
    "tiny_chunks": dict(B=3, H_Q=4, H_KV=2, d_h=8, block_size=4, kv_dtype="f32",
                        q_dtype="f32", layers=1, seed=5, lens="fixed_after",
                        lens_after_cfg=(8, 18, 34), new_tokens=(4, 1, 1), pool_blocks=32),
    "prefix_hit": dict(B=64, H_Q=32, H_KV=8, d_h=128, block_size=16, kv_dtype="bf16",
                       q_dtype="bf16", layers=1, seed=6, lens="prefix_chunk",
                       shared_tokens=1200, private_tokens=600),
}


@dataclass
class Workload:
    name: str
    B: int
    H_Q: int
    H_KV: int
    d_h: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    layers: int
    num_blocks: int
    max_blocks_per_seq: int
    block_table: torch.Tensor          # int32 [B, max_blocks_per_seq], -1 past the end
    context_lens: torch.Tensor         # int32 [B], after the append
    free_order: torch.Tensor           # int32 [num_blocks - used], ids not in any table
    shared_blocks: int                 # leading table entries shared by every request
    max_context_len: int               # max of context_lens (host value, for grid sizing)
    query_start: torch.Tensor = None   # int32 [B + 1], prefix sum of new tokens per request
    total_q: int = 0                   # new tokens in all (rows of q, k_new, v_new)
    max_q_len: int = 0                 # most new tokens of one request (host value)
    k_cache: list = field(default_factory=list)   # per layer [num_blocks, H_KV, bs, d_h]
    v_cache: list = field(default_factory=list)
    k_scale: list = field(default_factory=list)   # per layer fp32 [num_blocks, H_KV] (fp8 only)
    v_scale: list = field(default_factory=list)
    q: list = field(default_factory=list)         # per layer [total_q, H_Q, d_h]
    k_new: list = field(default_factory=list)     # per layer [total_q, H_KV, d_h]
    v_new: list = field(default_factory=list)

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_h)


def _draw_lens(cfg, B, gen):
    kind = cfg["lens"]
    if kind == "fixed":
        before = torch.tensor(cfg["lens_before"][:B], dtype=torch.int64)
        return before + 1
    if kind == "fixed_after":
        return torch.tensor(cfg["lens_after_cfg"][:B], dtype=torch.int64)
    if kind == "prefix_chunk":
        return torch.full((B,), cfg["shared_tokens"] + cfg["private_tokens"], dtype=torch.int64)
    if kind == "uniform":
        before = torch.randint(cfg["lo"], cfg["hi"] + 1, (B,), generator=gen)
        return before + 1
    if kind == "const_after":
        return torch.full((B,), cfg["n_after"], dtype=torch.int64)
    if kind == "shared":
        off = torch.randint(0, cfg["offset_hi"] + 1, (B,), generator=gen)
        return cfg["shared_tokens"] + cfg["private_tokens"] + off + 1
    if kind == "lognormal":
        z = torch.randn((B,), generator=gen, dtype=torch.float64)
        n = torch.round(cfg["median"] * torch.exp(z)).clamp(cfg["lo"], cfg["hi"])
        return n.to(torch.int64) + 1
    raise ValueError(kind)


def _ceil_div(a, b):
    return -(-a // b)


def make_workload(name: str, device="cpu", seed=None, values=True, **overrides) -> Workload:
    """Draw one decode step of the named workload on ``device``.

    ``overrides`` may change B, layers, H_KV, context lengths (``lens_after``
    as a list), new tokens per request (``new_tokens``, a list) and the pool
    factor (``pool_factor``) to make small variants for tests; everything
    else keeps the named workload's recipe.  ``values=False`` stops after
    the lengths and block tables (the pools, scales and new rows stay
    empty); the lengths and tables are the same as with values."""
    cfg = dict(CONFIGS[name])
    lens_after = overrides.pop("lens_after", None)
    new_tokens = overrides.pop("new_tokens", None)
    pool_factor = overrides.pop("pool_factor", 1.25)
    cfg.update(overrides)
    B, H_Q, H_KV, d_h, bs = cfg["B"], cfg["H_Q"], cfg["H_KV"], cfg["d_h"], cfg["block_size"]
    layers = cfg["layers"]
    gen = torch.Generator(device="cpu")
    gen.manual_seed(cfg["seed"] if seed is None else seed)

    # 1. context lengths (after the append)
    if lens_after is not None:
        lens = torch.tensor(list(lens_after), dtype=torch.int64)
        B = cfg["B"] = len(lens)
    else:
        lens = _draw_lens(cfg, B, gen)
    if new_tokens is None:
        new_tokens = cfg.get("new_tokens", 1)
        if cfg["lens"] == "prefix_chunk":
            new_tokens = cfg["private_tokens"]
    if isinstance(new_tokens, int):
        new_tokens = [new_tokens] * B
    new_tokens = [int(x) for x in new_tokens][:B]
    if len(new_tokens) != B or any(x < 0 or x > int(n) for x, n in zip(new_tokens, lens)):
        raise ValueError("need 0 <= new tokens <= context length for every request")
    qstart = torch.tensor([0] + new_tokens, dtype=torch.int64).cumsum(0)
    total_q = int(qstart[-1])
    nblk = [_ceil_div(int(n), bs) for n in lens]
    shared = (cfg.get("shared_tokens", 0) // bs
              if cfg["lens"] in ("shared", "prefix_chunk") else 0)
    needed = shared + sum(nb - shared for nb in nblk)
    num_blocks = cfg.get("pool_blocks") or max(_ceil_div(needed * int(pool_factor * 100), 100), needed)
    num_blocks = max(num_blocks, needed)
    max_blocks = max(nblk)

    # 2. physical ids: a random permutation dealt out in table order
    perm = torch.randperm(num_blocks, generator=gen).to(torch.int32)
    table = torch.full((B, max_blocks), -1, dtype=torch.int32)
    cursor = shared
    for b in range(B):
        table[b, :shared] = perm[:shared]
        k = nblk[b] - shared
        table[b, shared:nblk[b]] = perm[cursor:cursor + k]
        cursor += k
    free_order = perm[cursor:].clone()

    w = Workload(name=name, B=B, H_Q=H_Q, H_KV=H_KV, d_h=d_h, block_size=bs,
                 kv_dtype=cfg["kv_dtype"], q_dtype=cfg["q_dtype"], layers=layers,
                 num_blocks=num_blocks, max_blocks_per_seq=max_blocks,
                 block_table=table.to(device), context_lens=lens.to(torch.int32).to(device),
                 free_order=free_order, shared_blocks=shared,
                 max_context_len=int(lens.max().item()),
                 query_start=qstart.to(torch.int32).to(device), total_q=total_q,
                 max_q_len=max(new_tokens))

    if not values:
        return w
    # 3.. values, per layer, on the target device
    dgen = torch.Generator(device=device)
    dgen.manual_seed((cfg["seed"] if seed is None else seed) * 1000 + 17)
    pool_shape = (num_blocks, H_KV, bs, d_h)
    qt = _TORCH_DTYPE[cfg["q_dtype"]]
    for _ in range(layers):
        kf = torch.randn(pool_shape, generator=dgen, device=device, dtype=torch.float32)
        vf = torch.randn(pool_shape, generator=dgen, device=device, dtype=torch.float32)
        kn = torch.randn((total_q, H_KV, d_h), generator=dgen, device=device).to(qt)
        vn = torch.randn((total_q, H_KV, d_h), generator=dgen, device=device).to(qt)
        q = torch.randn((total_q, H_Q, d_h), generator=dgen, device=device).to(qt)
        if cfg["kv_dtype"] == "fp8_e4m3":
            ks = _fp8_scale(kf, kn)
            vs = _fp8_scale(vf, vn)
            kc = (kf / ks[:, :, None, None]).to(torch.float8_e4m3fn)
            vc = (vf / vs[:, :, None, None]).to(torch.float8_e4m3fn)
            w.k_scale.append(ks)
            w.v_scale.append(vs)
        else:
            kc = kf.to(_TORCH_DTYPE[cfg["kv_dtype"]])
            vc = vf.to(_TORCH_DTYPE[cfg["kv_dtype"]])
        del kf, vf
        w.k_cache.append(kc)
        w.v_cache.append(vc)
        w.k_new.append(kn)
        w.v_new.append(vn)
        w.q.append(q)
    return w


def _fp8_scale(pool_f32: torch.Tensor, new_vals: torch.Tensor) -> torch.Tensor:
    blk = pool_f32.abs().amax(dim=(2, 3))                       # [num_blocks, H_KV]
    new = new_vals.float().abs().amax(dim=(0, 2))               # [H_KV]
    m = torch.maximum(blk, new[None, :]).clamp_min(2.0 ** -120)
    return (m / 448.0).to(torch.float32)


def as_numpy(t: torch.Tensor):
    """CPU numpy view of a workload tensor: bf16 as uint16 bits, fp8 as uint8
    codes, everything else as is."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
