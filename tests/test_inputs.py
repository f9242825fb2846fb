"""The seeded input generator's paged pool (no GPU): every prefix position
sits at its block-table page and slot, and the reserve after each prefix is
mapped and zero."""
import numpy as np

import hydra_inputs as HI


def test_paged_pool_holds_prefixes_and_a_zero_reserve():
    w = HI.workload("tiny", B=3, L=(5, 40), scattered=True)
    for reserve in (None, 9):
        inp = HI.generate(w, reserve=reserve)
        r = w.n_heads + 1 if reserve is None else reserve
        bt = inp["block_table"].numpy()
        kp, vp = inp["k_pages"].numpy(), inp["v_pages"].numpy()
        ps = inp["page_size"]
        used = bt[bt >= 0]
        assert len(set(used.tolist())) == len(used) == kp.shape[0]  # every page mapped once
        for b, L in enumerate(inp["prefix_len"].tolist()):
            for p in range(L + r):
                page = bt[b, p // ps]
                assert page >= 0
                if p < L:
                    assert np.array_equal(kp[page, :, p % ps], inp["k_prefix"][b][p].numpy())
                    assert np.array_equal(vp[page, :, p % ps], inp["v_prefix"][b][p].numpy())
                else:
                    assert not kp[page, :, p % ps].any() and not vp[page, :, p % ps].any()
