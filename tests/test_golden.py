"""The oracle against the facts the pages print (tests/golden/page_facts.json)."""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic
from helpers import f64, global_pools
from test_oracle_ring import k_view

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def test_workload_shapes_match_the_pages():
    g = FACTS["global_key_count"]
    assert synthetic.GLOBAL_VERIFY.key_count == g["value"]
    assert synthetic.GLOBAL_VERIFY.S == FACTS["grouped_verify_rows"]["proposed_positions"]
    assert synthetic.GLOBAL_VERIFY.G == FACTS["grouped_verify_rows"]["q_heads_per_kv_head"]
    assert synthetic.GLOBAL_VERIFY.G * synthetic.GLOBAL_VERIFY.S == FACTS["grouped_verify_rows"]["rows"]
    assert (synthetic.GLOBAL_VERIFY.Hkv, synthetic.GLOBAL_VERIFY.D) == (
        FACTS["attention_shapes"]["global"]["kv_heads"], FACTS["attention_shapes"]["global"]["head_dim"])
    for w in (synthetic.SWA_DECODE, synthetic.SWA_VERIFY, synthetic.MIXED_SLIDING):
        assert w.W == FACTS["sliding_window"]["window"]
        assert (w.Hkv, w.D) == (FACTS["attention_shapes"]["sliding"]["kv_heads"],
                                FACTS["attention_shapes"]["sliding"]["head_dim"])
    assert synthetic.SWA_DECODE.B == FACTS["decode_batch"]["value"]


def test_padded_contraction_length_is_6016_for_6005_keys():
    # The oracle's padded form needs exactly pad64(6005) = 6016 slots: a region
    # of 6008 slots is refused, 6016 is accepted.
    g = FACTS["global_key_count"]
    kc, padded = g["value"], g["padded_to"]
    assert padded - kc == g["extra_columns"] and padded % g["pad_multiple"] == 0
    hkv, d = 1, 32
    k = synthetic.normal_bf16(synthetic.rng(3), (1, kc, hkv, d))
    q = synthetic.normal_bf16(synthetic.rng(4), (1, 1, 1, d))
    qp = np.array([[kc - 1]], np.int32)
    kcs = np.array([kc], np.int32)
    for cap, ok in ((padded - 8, False), (padded, True)):
        kp, vp, ko, vo = global_pools(k, k, kcs, cap)
        if ok:
            oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, qp, kcs, hkv, 0.3)
        else:
            with pytest.raises(ValueError):
                oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, qp, kcs, hkv, 0.3)


@pytest.mark.parametrize("pos,slot", [(1023, 1023), (1024, 0), (2500, 452), (4096, 0), (8191, 1023)])
def test_ring_slot_of_position_for_window_1024(pos, slot):
    W = FACTS["sliding_window"]["window"]
    hkv, d = 1, 32
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    kp, vp = np.zeros(rb, np.uint8), np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    one = synthetic.bf16_bits(np.ones((1, 1, hkv, d), np.float32))
    oracle.kv_append(kp, vp, off, off, W, oracle.BF16, 1, 1, one, one, np.array([pos], np.int32))
    K = f64(k_view(kp, 0, W, hkv, d))  # [slot][Hkv][D] through the declared layout
    assert list(np.nonzero(K[:, 0, 0])[0]) == [slot]
