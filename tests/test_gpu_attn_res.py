"""GPU parity of the attention-residual mixing against the fp64 oracle.

Every output element of small and ragged problems on every kernel path (the
streaming kernel that walks several tokens per workgroup with the next one
prefetched, one or two 128-bit vectors per lane with up to 12 or 16 blocks,
the two-pass element path for misaligned or very wide rows), bf16 and fp32 values / weights /
outputs, the split (stored sums + prefix) and stacked forms; sampled tokens at
the full Kimi-K3 width (8192 tokens x 9 blocks x 7168); determinism and token
independence.  Bound: ares_compare.py.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from ares_compare import assert_ares_close
from ref import host_f64, sample_rows, threads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ffn_gated_activation_amd  # noqa: F401


def _say(msg):
    print(msg, flush=True)


def _inputs(T, m, H, prefix=True, dt=torch.bfloat16, wdt=torch.bfloat16, seed=0, eps=1e-6):
    from ffn_gated_activation_amd.workloads import make_attn_res_inputs
    return make_attn_res_inputs(T, m, H, prefix=prefix, dtype=dt, w_dtype=wdt, device=DEV, seed=seed, eps=eps)


def _check(x, out_dtype=None, tokens=None, tag=""):
    from ffn_gated_activation_amd import situ_glu_attn_res_fwd
    blocks, prefix, w, p, eps = x["blocks"], x["prefix"], x["norm_weight"], x["proj_weight"], x["eps"]
    _say(f"[ares] {tag} blocks={None if blocks is None else tuple(blocks.shape)} prefix={prefix is not None} "
         f"{(blocks if blocks is not None else prefix).dtype} w={w.dtype} out={out_dtype}")
    out = situ_glu_attn_res_fwd(blocks, prefix, w, p, eps, out_dtype)
    torch.cuda.synchronize()
    if tokens is not None:
        idx = torch.as_tensor(tokens, device=DEV)
        blocks = None if blocks is None else blocks.index_select(0, idx)
        prefix = None if prefix is None else prefix.index_select(0, idx)
        out = out.index_select(0, idx)
    T = (blocks if blocks is not None else prefix).shape[0]
    H = w.numel()
    b64 = host_f64(blocks) if blocks is not None else np.zeros((T, 0, H))
    ref = oracle.attn_res_forward(b64, None if prefix is None else host_f64(prefix), host_f64(w), host_f64(p), eps,
                                  threads=threads())
    nb = b64.shape[1] + (prefix is not None)
    st = assert_ares_close(tag, out, ref, nb)
    _say(f"[ares] {tag} ok {st}")
    return out


CASES = [
    # T, m, H, prefix, values, weights, out   (path)
    (64, 8, 7168, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),      # Kimi-K3 width, 9 blocks (1)
    (33, 3, 1024, True, torch.float32, torch.float32, torch.bfloat16),        # fp32 values (1)
    (17, 12, 512, True, torch.bfloat16, torch.float32, torch.float32),        # 13 blocks (3)
    (9, 4, 12288, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),      # two vectors per lane (2)
    (5, 2, 1000, True, torch.bfloat16, torch.bfloat16, torch.float32),        # ragged strip (1)
    (7, 5, 1003, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),       # odd width: element path
    (6, 16, 256, False, torch.bfloat16, torch.bfloat16, torch.bfloat16),      # 16 blocks, stacked (3)
    (4, 9, 7168, True, torch.float32, torch.bfloat16, torch.float32),         # fp32, 10 blocks, 1792 vectors (0)
    (3, 1, 20000, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),      # very wide: element path
    (8, 0, 4096, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),       # prefix only: one block
    (8, 1, 64, False, torch.float32, torch.float32, torch.float32),           # one stacked block
    (700, 8, 2048, True, torch.bfloat16, torch.bfloat16, torch.bfloat16),     # streaming: 2 or 3 tokens per workgroup
    (513, 4, 512, True, torch.bfloat16, torch.float32, torch.bfloat16),       # streaming, 5 blocks
]


@pytest.mark.parametrize("T,m,H,prefix,dt,wdt,odt", CASES)
def test_small(T, m, H, prefix, dt, wdt, odt):
    x = _inputs(T, m, H, prefix, dt, wdt, seed=T + m)
    _check(x, odt, tag=f"T{T} m{m} H{H}")


@pytest.mark.parametrize("nb", range(1, 11))
def test_stream_every_block_count(nb):
    # the streaming kernel has one instantiation per block count 1..10
    x = _inputs(300, nb - 1, 1024, True, torch.bfloat16, torch.bfloat16, seed=40 + nb)
    _check(x, torch.bfloat16, tag=f"stream nb={nb}")


def test_eps_zero_and_large():
    for eps in (0.0, 1.0):
        _check(_inputs(16, 6, 2048, True, eps=eps, seed=3), tag=f"eps={eps}")


def test_misaligned_element_path():
    x = _inputs(5, 3, 768, True, seed=4)
    flat = torch.empty(x["blocks"].numel() + 1, dtype=x["blocks"].dtype, device=DEV)
    b = flat[1:].view(x["blocks"].shape)
    b.copy_(x["blocks"])
    x["blocks"] = b
    _check(x, tag="misaligned blocks")


def test_peaked_and_flat_softmax():
    x = _inputs(12, 8, 1024, True, seed=5)
    x["proj_weight"] = x["proj_weight"] * 40.0      # one block dominates most tokens
    _check(x, tag="peaked")
    x["proj_weight"] = torch.zeros_like(x["proj_weight"])  # the mean of the blocks
    _check(x, tag="flat")


def test_full_size_sampled():
    from ffn_gated_activation_amd.workloads import ATTN_RES, make_attn_res_inputs
    w = ATTN_RES["attn_res_mix"]
    x = make_attn_res_inputs(w.tokens, w.stored, w.hidden, True, device=DEV, seed=0, eps=w.eps)
    _check(x, tokens=sample_rows(w.tokens, k=40), tag="attn_res_mix full")


def test_split_equals_stacked_and_deterministic():
    from ffn_gated_activation_amd import apply_attn_res, attn_res_core, situ_glu_attn_res_fwd
    x = _inputs(40, 5, 2048, True, seed=6)
    a = situ_glu_attn_res_fwd(x["blocks"], x["prefix"], x["norm_weight"], x["proj_weight"], x["eps"])
    b = situ_glu_attn_res_fwd(x["blocks"], x["prefix"], x["norm_weight"], x["proj_weight"], x["eps"])
    values = torch.cat([x["blocks"], x["prefix"].unsqueeze(1)], dim=1).contiguous()
    c = attn_res_core(values, x["norm_weight"], x["proj_weight"], x["eps"], torch.bfloat16)
    d = apply_attn_res(x["prefix"], x["blocks"], x["norm_weight"], x["proj_weight"], x["eps"])
    sub = situ_glu_attn_res_fwd(x["blocks"][10:20].contiguous(), x["prefix"][10:20].contiguous(),
                                x["norm_weight"], x["proj_weight"], x["eps"])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c) and torch.equal(a, d)
    assert torch.equal(a[10:20], sub)


def test_empty():
    from ffn_gated_activation_amd import situ_glu_attn_res_fwd
    w = torch.ones(64, device=DEV, dtype=torch.bfloat16)
    out = situ_glu_attn_res_fwd(torch.zeros(0, 3, 64, device=DEV, dtype=torch.bfloat16), None, w, w, 1e-6)
    assert out.shape == (0, 64)
