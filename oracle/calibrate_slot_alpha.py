"""Find the Zipf bias strength alpha of the slot-table workload.

The pages report that keeping roughly a quarter of the experts resident on
the GPU gives a hit rate of about 70 % ([JD] section "为什么从 18t/s 变成
60-90t/s"; [AF] section "命中率七成，代价是答案会变").  The slot-table
workload keeps the 128 most popular of 512 experts resident and draws logits
N(0,1) + alpha * log p_r with Zipf exponent 1.2.  This script bisects alpha
so that the mean share of routed (token, rank) pairs that hit is 0.70, using
the oracle's router, and prints it; the value is stored in
``synth.SLOT_ALPHA``.

Run: python -m oracle.calibrate_slot_alpha
"""
import numpy as np

import synth
from oracle.moe_oracle import route


def hit_rate(alpha, layers=48, tokens=64, E=512, k=10, resident=128, s=synth.SLOT_ZIPF_S):
    hits = 0
    for layer in range(layers):
        lg = synth.router_logits(1000 + 0, layer, tokens, E, zipf_s=s, alpha=alpha)
        idx, _ = route(lg, k)
        ranks = synth.expert_ranks(1000 + 0, layer, E)
        hits += np.count_nonzero(ranks[idx] <= resident)
    return hits / (layers * tokens * k)


def main():
    lo, hi = 0.0, 2.0
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        if hit_rate(mid) < 0.70:
            lo = mid
        else:
            hi = mid
    a = round(0.5 * (lo + hi), 3)
    print("alpha = %.3f  hit rate = %.4f" % (a, hit_rate(a)))


if __name__ == "__main__":
    main()
