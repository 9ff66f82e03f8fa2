"""The quantizer variant selection rule (host logic, pure, no GPU).

Pinned to the page "fp8_act_quant_floor.rs" (spark_model/layers/ops):
parameterised with that page's H100 numbers (132 SMs, floor of 2 workgroups
per SM, 8 K-groups per workgroup of the K-grouped variant) the rule must
reproduce the per-K threshold table of the module header ("The rule") and
the winner of all fifteen measured arms ("The defect this closes"), test the
guards in the page's order (fp8_act_quant_hopper_reject) and map verdicts to
log slots as fp8_quant_log_slot does.  The stored numbers are in
tests/golden/floor_table_h100.txt.
"""
import os

import pytest

import w8a8_fp8_block_amd as fp8q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "floor_table_h100.txt")


def _golden():
    A, B, C = [], [], {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        if f[0] == "A":
            A.append(tuple(int(v) for v in f[1:]))
        elif f[0] == "B":
            B.append((int(f[1]), int(f[2]), f[5]))
        elif f[0] == "C":
            C[f[1]] = int(f[2])
    return A, B, C


def _h100(requested=1, b=1, a=1):
    _, _, C = _golden()
    return fp8q.SelectParams(C["sm_count"], C["min_ctas_per_sm"], C["groups_per_cta"], 1,
                             requested, b, a)


def test_h100_threshold_table():
    A, _, _ = _golden()
    p = _h100()
    assert len(A) == 3
    for K, G, gy, min_m in A:
        assert K // 128 == G
        assert fp8q.fp8q_quant_b_min_m(K, p) == min_m
        v, grid, why = fp8q.fp8q_quant_select_with(min_m, K, p)
        assert v == 2 and why is None and grid == (min_m, gy, 1)
        v, _, why = fp8q.fp8q_quant_select_with(min_m - 1, K, p)
        assert v == 1 and why == "too few workgroups for variant B to fill the device"


def test_h100_reproduces_all_fifteen_arm_winners():
    _, B, _ = _golden()
    p = _h100()
    assert len(B) == 15
    for M, K, winner in B:
        v, _, _ = fp8q.fp8q_quant_select_with(M, K, p)
        assert v == (2 if winner == "twin" else 1), (M, K, winner)


def test_h100_prefill_margin():
    """M=1168 clears every per-K threshold by 22x to 73x (module header)."""
    A, _, _ = _golden()
    ratios = [1168 / min_m for _, _, _, min_m in A]
    assert int(min(ratios)) == 22 and int(max(ratios)) == 73


def test_reject_order():
    # B absent beats everything, even a missing A
    assert fp8q.fp8q_quant_select_with(10000, 5120, _h100(b=0))[2] == "variant B absent"
    # A absent: B runs even when not requested and below the floor
    v, _, why = fp8q.fp8q_quant_select_with(1, 5120, _h100(requested=0, a=0))
    assert v == 2 and why is None
    # not requested is tested before the floor
    assert fp8q.fp8q_quant_select_with(1, 5120, _h100(requested=0))[2] == "variant B not requested"
    assert fp8q.fp8q_quant_select_with(10000, 5120, _h100(requested=0))[2] == "variant B not requested"
    # neither present / bad K -> -1
    assert fp8q.fp8q_quant_select_with(16, 5120, _h100(b=0, a=0))[0] == -1
    assert fp8q.fp8q_quant_select_with(16, 5000, _h100())[0] == -1


def test_variant_a_grid():
    p = _h100()
    v, grid, why = fp8q.fp8q_quant_select_with(16, 5120, p)
    assert v == 1 and grid == (16 * 40, 1, 1)  # one group per workgroup in this parameterisation


def test_log_slots():
    R = ["variant B not requested", "variant B absent",
         "too few workgroups for variant B to fill the device"]
    assert fp8q.fp8q_quant_log_slot(2, None, True) == 3
    assert fp8q.fp8q_quant_log_slot(2, None, False) == 3
    for i, r in enumerate(R):
        assert fp8q.fp8q_quant_log_slot(1, r, True) == i
        assert fp8q.fp8q_quant_log_slot(1, r, False) == -1  # lever off: silence
    # replay of a serve's call order: one line per slot
    seen = []
    p = _h100()
    for M in (27, 1168, 16, 4576, 25):
        v, _, why = fp8q.fp8q_quant_select_with(M, 5120, p)
        s = fp8q.fp8q_quant_log_slot(v, why, True)
        if s >= 0 and s not in seen:
            seen.append(s)
    assert seen == [2, 3]


def test_gfx950_defaults_are_consistent():
    p = fp8q.fp8q_default_select_params(256)
    assert p.cu_count == 256 and p.min_wg_per_cu >= 1 and p.b_groups_per_wg >= 1
    for K in (5120, 6144, 17408):
        mm = fp8q.fp8q_quant_b_min_m(K, p)
        assert mm >= 1
        if p.requested:
            assert fp8q.fp8q_quant_select(mm, K, 256)[0] == 2
            if mm > 1:
                assert fp8q.fp8q_quant_select(mm - 1, K, 256)[0] == 1
