"""Host-side logic that needs no GPU: the output tolerance rule of the parity tests."""
import numpy as np
import torch

from cases import half_ulp_bf16, output_bound


def test_half_ulp_is_half_the_bf16_spacing():
    # spacing of bf16 at x: the next bf16 value up minus x, for x a bf16 value (computed with torch's bf16)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 5, 2000), [1.0, 1.5, 8.0, 2688.0]])
    xb = torch.from_numpy(np.abs(x).astype(np.float32)).to(torch.bfloat16)
    nxt = (xb.view(torch.int16) + 1).view(torch.bfloat16)
    spacing = (nxt.double() - xb.double()).numpy()
    np.testing.assert_array_equal(half_ulp_bf16(xb.double().numpy()), spacing / 2)


def test_output_bound_adds_at_most_2_pow_minus_6_below_8():
    v = np.linspace(-7.999, 7.999, 10001)
    assert output_bound(v).max() <= 2e-2 + 2.0 ** -6
    assert output_bound(np.array([0.0]))[0] == 2e-2 + 2.0 ** -134
    assert output_bound(np.array([2688.0]))[0] == 2e-2 + 8.0  # bf16 spacing 16 in [2048, 4096)


def test_v_abs_of_rows_matches_the_oracle_dequant():
    import oracle
    import workloads as W
    from cases import v_abs_of_rows
    rng = np.random.default_rng(8)
    lat, rope = W.gen_latent_rope(rng, 20)
    for fmt, quant, deq in (("nvfp4", oracle.quant_row_nvfp4, oracle.dequant_row_nvfp4),
                            ("fp8", oracle.quant_row_fp8, oracle.dequant_row_fp8)):
        rows = np.stack([quant(lat[i], rope[i]) for i in range(20)])
        ref = np.abs(np.stack([deq(r)[:512] for r in rows]))
        np.testing.assert_array_equal(v_abs_of_rows(rows, fmt), ref)
