"""Pins of the oracle's FLOP accounting against the pages' printed numbers.

The Mistral benchmark page (breakdown items 10-11) gives the slow and fast
costs of the LoRA gradient chain, (h d)(m + r) and (m r)(h + d), and prints the
large-m ratios 186.58 (Llama 7b) and 398.22 (Llama 70b); both are stored in
tests/golden/bracketing_ratios.txt with that citation.
"""
import os

from oracle import qlora as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bracketing_ratios.txt")


def test_chain_costs_are_the_pages_closed_forms():
    for m, d, h, r in ((8192, 4096, 11008, 16), (16384, 8192, 28672, 64), (7, 3, 5, 2)):
        _, slow, fast = Q.lora_grad_bracketing_ratio(m, d, h, r)
        assert slow == h * d * (m + r)
        assert fast == m * r * (h + d)


def test_large_m_ratio_reproduces_printed_values():
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 2
    for _, h, d, r, printed in rows:
        ratio, _, _ = Q.lora_grad_bracketing_ratio(10 ** 12, int(d), int(h), int(r))
        assert f"{ratio:.2f}" == printed


def test_mlp_flops_count_six_base_products():
    m, d, h, r = 8192, 4096, 11008, 16
    f = Q.mlp_algorithmic_flops(m, d, h, r)
    # each base product is 2*m*d*h; the LoRA share is under 1%
    assert 6 * 2 * m * d * h < f < 1.01 * 6 * 2 * m * d * h
    assert f == 4468041056256
