"""The router's logit kernels reproduce the fixed float32 order bit for bit on
adversarial operands.

The logit order is one fused multiply-add chain per (token, expert) over k
ascending from +0 (the pages leave the order open; the library fixes this
one so that routing is bit exact).  The large-router kernel runs it on the
float32 matrix cores, as chains of 16x16x4 multiply-accumulates over
ascending k-quads; that each such instruction adds its four products one at
a time, each with one rounding, is a measured property of the hardware, not
a documented one.  These tests pin it (and the VALU kernels) through
``moe_route`` on operands built to separate the fmaf chain from every other
plausible summation:

* products that are not float32 numbers (bf16 x times full-mantissa float32
  W), so a separate multiply and add would round twice;
* exact products (power-of-two weights) and quads led by an element 2^24
  times larger than the rest, so that running sums often tie or round at
  each step where a wider sum of the quad would not;
* subnormal products and subnormal running sums;
* signed zeros (zero operands, and products that cancel the sum exactly);
* exponent spreads beyond 2^50 inside one chain (absorption, cancellation).

Before the GPU comparison, each case checks on the CPU that its operands do
separate the fmaf chain from a chain with separately rounded multiply and
add, and from quads summed in float64 and rounded once, on a sizeable share of
the logits: a kernel with another order would fail the comparison.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_mixture_experts_renormalised_amd import binding
    binding.lib()
    yield


def bf16_round(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32)))


def adversarial_operands(T, N, d, seed, dtype):
    """x [T, d] (bf16-representable for bf16 layers) and W [N, d] float32."""
    rng = np.random.default_rng(seed)
    # W: random signs, exponents over 2^-24 .. 2^2, half exact powers of two
    # (exact products, so sums tie often) and half full 24-bit mantissas
    # (products that are not float32 numbers); zero entries of either sign;
    # some rows scaled by 2^-105 (subnormal products with small tokens); a few
    # rows of -0 (their logits are +0: the chain starts at +0)
    wexp = rng.integers(-24, 3, size=(N, d))
    wman = np.where(rng.random((N, d)) < 0.5, 1.0,
                    1.0 + rng.integers(0, 1 << 23, (N, d)) / 2.0**23)
    w = np.where(rng.random((N, d)) < 0.5, -1.0, 1.0) * wman * np.exp2(wexp.astype(np.float64))
    w[rng.random((N, d)) < 0.03] = 0.0
    w[rng.random((N, d)) < 0.02] = -0.0
    w[rng.random(N) < 0.15] *= 2.0**-105
    w[rng.choice(N, size=max(1, N // 20), replace=False)] = -0.0
    w = w.astype(np.float32)
    # x: 8-bit mantissas over 2^-8 .. 2^8, zeros of either sign, bf16
    # subnormals (2^-133 .. 2^-127), tokens scaled by 2^-30 (with the small W
    # rows their products and sums are subnormal), a few all-zero tokens, and
    # tokens with one large leading element per quad (2^24 times the rest):
    # the later products of the quad are then near half an ulp of the sum
    xexp = rng.integers(-8, 9, size=(T, d))
    xman = 1.0 + rng.integers(0, 128, (T, d)) / 128.0
    x = np.where(rng.random((T, d)) < 0.5, -1.0, 1.0) * xman * np.exp2(xexp.astype(np.float64))
    x[rng.random((T, d)) < 0.04] = 0.0
    x[rng.random((T, d)) < 0.02] = -0.0
    sub = rng.random((T, d)) < 0.02
    x[sub] = rng.integers(1, 128, sub.sum()) * 2.0**-133 * np.where(rng.random(sub.sum()) < 0.5, -1, 1)
    x[rng.random(T) < 0.2] *= 2.0**-30
    lead = rng.random(T) < 0.3
    x[np.ix_(lead, np.arange(0, d, 4))] *= 2.0**24
    zero_tok = rng.choice(T, size=max(1, T // 50), replace=False)
    x[zero_tok] = np.where(rng.random((zero_tok.size, d)) < 0.5, 0.0, -0.0)
    if dtype == "bf16":
        x = bf16_round(x)
    return x.astype(np.float32), w


def fmaf_chain(x, w):
    """Reference: the oracle's fixed-order logits (C fmaf chain)."""
    return oracle.router_logits(x, w, None)


def separate_chain(x, w):
    """float32 chain with the product rounded before the add (not the library's order)."""
    acc = np.zeros((x.shape[0], w.shape[0]), dtype=np.float32)
    for k in range(x.shape[1]):
        p = np.multiply.outer(x[:, k], w[:, k]).astype(np.float32)
        acc = (acc + p).astype(np.float32)
    return acc


def wide_quad_chain(x, w):
    """Each k-quad's four products added to the running sum in float64, then
    rounded once to float32 (a wider in-instruction sum; not the library's
    order)."""
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    acc = np.zeros((x.shape[0], w.shape[0]), dtype=np.float32)
    for q in range(0, x.shape[1], 4):
        s = acc.astype(np.float64)
        for j in range(q, min(q + 4, x.shape[1])):
            s = s + np.multiply.outer(x64[:, j], w64[:, j])
        acc = s.astype(np.float32)
    return acc


CASES = [
    # (name, T, N, d, dtype): one-logit-per-lane kernel (scalar W), the three
    # launch shapes of the matrix-core kernel, and the float32 VALU kernel
    ("sw_valu", 70, 40, 256, "bf16"),
    ("mfma_64x16", 9000, 12, 128, "bf16"),
    ("mfma_32x32", 1500, 100, 192, "bf16"),
    ("mfma_64x64", 2100, 272, 320, "bf16"),
    ("f32_valu", 300, 48, 96, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_router_chain_bit_exact_on_adversarial_operands(case):
    from sparse_mixture_experts_renormalised_amd import binding as B
    name, T, N, d, dtype = case
    print(f"[router-chain] {name}: T={T} N={N} d={d} {dtype}", flush=True)
    x, w = adversarial_operands(T, N, d, seed=len(name) * 1009 + T, dtype=dtype)
    ref = fmaf_chain(x, w)
    bits = ref.view(np.uint32)
    # the operands discriminate: other orders give other bits on many logits
    sep = separate_chain(x, w).view(np.uint32)
    quad = wide_quad_chain(x, w).view(np.uint32)
    assert np.mean(sep != bits) > 0.05, np.mean(sep != bits)
    assert np.mean(quad != bits) > 0.05, np.mean(quad != bits)
    # subnormal and signed-zero logits occur
    assert np.any((ref != 0) & (np.abs(ref) < np.finfo(np.float32).tiny))
    assert np.any(bits == 0)
    K = min(8, N)
    cfg = B.config(T, d, N, K, 0, 64, dtype)
    xt = torch.from_numpy(x)
    xd = (xt.to(torch.bfloat16) if dtype == "bf16" else xt).cuda()
    assert torch.equal(xd.float().cpu(), xt)          # x is exactly representable
    wd = torch.from_numpy(w).cuda()
    logits = torch.empty((T, N), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    gates = torch.empty((T, K), dtype=torch.float32, device="cuda")
    B.route(cfg, xd, wd, None, logits, idx, gates)
    torch.cuda.synchronize()
    got = logits.cpu().numpy().view(np.uint32)
    bad = np.nonzero(got != bits)
    assert bad[0].size == 0, (f"{bad[0].size} logits differ, first at {bad[0][0]},{bad[1][0]}: "
                              f"{got[bad][0]:#010x} vs {bits[bad][0]:#010x}")
