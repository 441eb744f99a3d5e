"""Pins of the oracle's attention over fp8 caches.

Page 2, "KV Cache Explained", section "What changes when you use FP8 KV":
FP8 stores one byte per element and the quantized values need scales.  The
cache format here is OCP E4M3 codes with one float32 scale per (physical
block, KV head), separately for K and for V; a stored element means
code value x scale.  The oracle's ``gather_head`` applies that rule while it
walks the block table.

The checks below do not go through the oracle's codec or gather: the codes
are decoded by torch's float8_e4m3fn conversion (a library routine), each
position is looked up by hand in the table, multiplied by the scale of its
own block and head, and the dense K and V go through torch's float64
scaled_dot_product_attention.  K and V get different random scales for
every (block, head), so a swapped pair of scales, a scale taken from the
wrong head or from the wrong block changes the result by far more than the
1e-12 tolerance; the last test shows that it does, by passing the oracle
exactly such wrong scales.
"""

import numpy as np
import pytest
import torch

from oracle import paged

BS = 16


def _fp8_case(H_Q, H_KV, lens, d=32, seed=0):
    rng = np.random.default_rng(seed)
    nblk = [-(-n // BS) for n in lens]
    num_blocks = sum(nblk) + 7                     # a few blocks no table maps
    perm = rng.permutation(num_blocks)
    table = np.full((len(lens), max(nblk)), -1, dtype=np.int32)
    c = 0
    for b, k in enumerate(nblk):
        table[b, :k] = perm[c:c + k]
        c += k
    # codes of magnitude <= 3.75 (exponent field <= 8), random sign; every
    # slot holds a finite code, used or not
    shape = (num_blocks, H_KV, BS, d)
    mag = rng.integers(0, 0x48, size=shape, dtype=np.uint8)
    sign = (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7).astype(np.uint8)
    kc = mag | sign
    mag = rng.integers(0, 0x48, size=shape, dtype=np.uint8)
    sign = (rng.integers(0, 2, size=shape, dtype=np.uint8) << 7).astype(np.uint8)
    vc = mag | sign
    # independent scales for K and V, for every (block, head)
    k_scale = (2.0 ** rng.uniform(-3, 1, size=(num_blocks, H_KV))).astype(np.float32)
    v_scale = (2.0 ** rng.uniform(-3, 1, size=(num_blocks, H_KV))).astype(np.float32)
    q = torch.randn((len(lens), H_Q, d), generator=torch.Generator().manual_seed(seed),
                    dtype=torch.float32).to(torch.bfloat16)
    q_bits = q.view(torch.int16).numpy().view(np.uint16)
    return dict(q_bits=q_bits, q=q.to(torch.float64), kc=kc, vc=vc, k_scale=k_scale,
                v_scale=v_scale, table=table, lens=list(lens), H_Q=H_Q, H_KV=H_KV, d=d)


def _reference(c, scale):
    """Library decode + hand gather + torch float64 SDPA: [B, H_Q, d]."""
    kdec = torch.from_numpy(c["kc"]).view(torch.float8_e4m3fn).to(torch.float64)
    vdec = torch.from_numpy(c["vc"]).view(torch.float8_e4m3fn).to(torch.float64)
    g = c["H_Q"] // c["H_KV"]
    out = []
    for b, n in enumerate(c["lens"]):
        K = torch.empty((c["H_KV"], n, c["d"]), dtype=torch.float64)
        V = torch.empty_like(K)
        for t in range(n):
            p = int(c["table"][b][t // BS])
            r = t % BS
            for h in range(c["H_KV"]):
                K[h, t] = kdec[p, h, r] * float(c["k_scale"][p, h])
                V[h, t] = vdec[p, h, r] * float(c["v_scale"][p, h])
        Kt = K.repeat_interleave(g, dim=0)[None]
        Vt = V.repeat_interleave(g, dim=0)[None]
        qt = c["q"][b][None, :, None, :]
        o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
        out.append(o[0, :, 0, :])
    return torch.stack(out).numpy()


def _oracle(c, scale, k_scale=None, v_scale=None):
    return paged.attend(c["q_bits"], "bf16", c["kc"], c["vc"], "fp8_e4m3", c["table"],
                        np.asarray(c["lens"]), BS, scale,
                        c["k_scale"] if k_scale is None else k_scale,
                        c["v_scale"] if v_scale is None else v_scale)


# MQA (one KV head for all query heads), GQA and MHA, with lengths that end
# inside a block, on a block boundary and at one position
SHAPES = [(8, 1, [1, 16, 40]), (8, 2, [17, 33, 5]), (4, 4, [48, 7, 21])]


@pytest.mark.parametrize("H_Q,H_KV,lens", SHAPES, ids=["mqa", "gqa", "mha"])
def test_fp8_attention_matches_library_decode_and_sdpa(H_Q, H_KV, lens):
    c = _fp8_case(H_Q, H_KV, lens, seed=H_KV)
    scale = 1.0 / np.sqrt(c["d"])
    out = _oracle(c, scale)
    ref = _reference(c, scale)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_fp8_attention_with_power_of_two_scales_equals_f32_cache():
    # with power-of-two scales every code x scale is a float32, so an f32
    # cache holding the library-decoded values must give the same output
    c = _fp8_case(8, 2, [23, 50], seed=7)
    rng = np.random.default_rng(8)
    c["k_scale"] = (2.0 ** rng.integers(-4, 3, size=c["k_scale"].shape)).astype(np.float32)
    c["v_scale"] = (2.0 ** rng.integers(-4, 3, size=c["v_scale"].shape)).astype(np.float32)
    kdec = torch.from_numpy(c["kc"]).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    vdec = torch.from_numpy(c["vc"]).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    k32 = kdec * c["k_scale"][:, :, None, None]
    v32 = vdec * c["v_scale"][:, :, None, None]
    scale = 0.3
    out8 = _oracle(c, scale)
    out32 = paged.attend(c["q_bits"], "bf16", k32, v32, "f32", c["table"], np.asarray(c["lens"]),
                         BS, scale)
    assert np.max(np.abs(out8 - out32)) < 1e-12


def test_wrong_scales_are_caught():
    # the reference above separates the plausible scale mistakes: K and V
    # scales swapped, the scale of the next KV head, the scale of another block
    c = _fp8_case(8, 2, [33, 40, 18], seed=3)
    scale = 1.0 / np.sqrt(c["d"])
    ref = _reference(c, scale)
    ks, vs = c["k_scale"], c["v_scale"]
    wrong = {
        "swapped": (vs, ks),
        "next_head": (np.roll(ks, 1, axis=1), np.roll(vs, 1, axis=1)),
        "next_block": (np.roll(ks, 1, axis=0), np.roll(vs, 1, axis=0)),
        "v_only_swapped_heads": (ks, np.roll(vs, 1, axis=1)),
    }
    for name, (k_s, v_s) in wrong.items():
        err = np.max(np.abs(_oracle(c, scale, k_s, v_s) - ref))
        assert err > 1e-3, name
