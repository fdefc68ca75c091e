"""The combine's parity bar where its terms cancel (no GPU needed).

The oracle rounds the exact weighted sum once; the GPU accumulates
w_k * y_k in fp32 with one rounding per fused multiply-add, in k order,
then rounds to bf16. With terms of mixed sign (a grouped GEMM's outputs,
"Enabling trillion-parameter models on AWS EFA", section "Dispatch and
combine") the fp32 accumulation error can exceed one bf16 ulp of a small
result, so a bar relative to |o| alone is not sound. These checks emulate
the fp32 accumulation on the CPU (numpy, exact products, the sum rounded via
float64 then float32) and show that the bar of combine_close holds where
the relative one fails.
"""
import numpy as np
import torch

import ep_workloads as W
import oracle
from gpu_util import abs_term_sum, bf16_close, combine_close, random_bf16


def fp32_fma_chain(w, y):
    """acc = fl32(w_k * y_k + acc) for k ascending from +0, then bf16 RNE.
    w: fp32 [T, R]; y: bf16 bits [T, R, H]."""
    acc = np.zeros((y.shape[0], y.shape[2]), np.float32)
    for k in range(y.shape[1]):
        prod = w[:, k, None].astype(np.float64) * W.bf16_bits_to_f32(y[:, k]).astype(np.float64)
        acc = (acc.astype(np.float64) + prod).astype(np.float32)
    return W.to_bf16_bits(acc)


def oracle_tokens(w, y):
    return np.stack([oracle.combine_token(w[t], [y[t, k] for k in range(y.shape[1])])
                     for t in range(y.shape[0])])


def test_bar_holds_where_the_relative_bar_fails():
    rng = np.random.default_rng(21)
    T, R, H = 256, 8, 1024
    w = rng.dirichlet(np.ones(R), size=T).astype(np.float32)
    y = random_bf16(rng, (T, R, H))
    # make the last term cancel the first seven almost exactly in half the
    # tokens: y_7 = bf16(-sum_{k<7} w_k y_k / w_7)
    head = (w[:, :7, None].astype(np.float64) *
            W.bf16_bits_to_f32(y[:, :7]).astype(np.float64)).sum(1)
    half = T // 2
    y[:half, 7] = W.to_bf16_bits((-head[:half] / w[:half, 7, None]).astype(np.float32))
    g = fp32_fma_chain(w, y)
    o = oracle_tokens(w, y)
    S = abs_term_sum(w, y)
    assert combine_close(g, o, S, R).all()
    assert not bf16_close(g, o).all()            # cancellation really happens here
    # the absolute term stays below one bf16 ulp of |o| unless |o| << S
    big = np.abs(W.bf16_bits_to_f32(o)) > 2.0 ** -12 * S
    assert bf16_close(g[big], o[big]).all()


def test_exact_cancellation_of_equal_weight_pairs():
    """w_{2i} = w_{2i+1}, y_{2i+1} = -y_{2i}: the exact sum is 0 (oracle +0),
    the fp32 chain leaves the rounding error of a product."""
    rng = np.random.default_rng(22)
    T, R, H = 64, 8, 512
    w = np.repeat(rng.dirichlet(np.ones(R // 2), size=T) / 2, 2, axis=1).astype(np.float32)
    y = random_bf16(rng, (T, R, H))
    y[:, 1::2] = y[:, 0::2] ^ np.uint16(0x8000)
    o = oracle_tokens(w, y)
    assert (o == 0).all()
    g = fp32_fma_chain(w, y)
    assert combine_close(g, o, abs_term_sum(w, y), R).all()


def test_bar_is_not_loose_for_same_sign_terms():
    """Positive terms: the bar is the relative one (plus under 2^-20 of it)."""
    rng = np.random.default_rng(23)
    T, R, H = 128, 8, 512
    w = rng.dirichlet(np.ones(R), size=T).astype(np.float32)
    y = random_bf16(rng, (T, R, H)) & np.uint16(0x7FFF)
    g = fp32_fma_chain(w, y)
    o = oracle_tokens(w, y)
    S = abs_term_sum(w, y)
    assert bf16_close(g, o).all()
    absolute = 2.0 * R * 2.0 ** -24 * S
    assert (absolute <= 2.0 ** -19 * np.abs(W.bf16_bits_to_f32(o))).all()


def test_torch_bf16_cast_is_round_to_nearest_even():
    """fp32_fma_chain's last step (torch's cast) rounds ties to even."""
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], np.float32)
    assert W.to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0xBF80]
    assert torch.tensor(1 + 2 ** -8).to(torch.bfloat16).item() == 1.0
