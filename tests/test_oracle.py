"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import pins


@pytest.fixture(scope="module")
def O():
    return pins.real_oracle()


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(O, check):
    fails = check(O)
    assert not fails, fails


def test_oracle_decode_step_small_case_matches_brute_force():
    """The step runner (cache fill through the block table, append at the
    prefill position, attention) agrees with brute force on logical rows."""
    import dataclasses

    import workloads
    from oracle import brute, mfa, run
    w = dataclasses.replace(workloads.WORKLOADS[3], batch=3, heads=2, head_dim=4,
                            context_range=(60, 70))
    inp = workloads.make_inputs(3, workload=w)
    res = run.decode_step(inp)
    for b in range(3):
        k, v = run.sequence_tokens(inp, b)
        kf, vf = mfa.bf16_bits_to_f64(k), mfa.bf16_bits_to_f64(v)
        assert kf.shape[0] == inp["seq_lens"][b]
        q = mfa.bf16_bits_to_f64(inp["q"][b])
        want = brute.attention(q.tolist(), kf.tolist(), vf.tolist(), 0.5)
        np.testing.assert_allclose(res["o"][b], want, rtol=1e-12, atol=1e-13)


def test_oracle_fp8_step_uses_dequantised_cache():
    import dataclasses

    import workloads
    from oracle import brute, e4m3, mfa, run
    w = dataclasses.replace(workloads.WORKLOADS[4], batch=2, heads=2, head_dim=8, context=70)
    inp = workloads.make_inputs(4, workload=w)
    res = run.decode_step(inp)
    for b in range(2):
        k, v = run.sequence_tokens(inp, b)
        kc, ks = mfa.quantize_tokens(mfa.bf16_bits_to_f64(k))
        vc, vs = mfa.quantize_tokens(mfa.bf16_bits_to_f64(v))
        kd = e4m3.decode(kc) * ks[:, None].astype(np.float64)
        vd = e4m3.decode(vc) * vs[:, None].astype(np.float64)
        q = mfa.bf16_bits_to_f64(inp["q"][b])
        want = brute.attention(q.tolist(), kd.tolist(), vd.tolist(), 1 / np.sqrt(8))
        np.testing.assert_allclose(res["o"][b], want, rtol=1e-12, atol=1e-13)
