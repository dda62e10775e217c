"""The MoE tail on the GPU (through the C-ABI): residual add + RMSNorm, alone
(moe_residual_rmsnorm) and fused into the combine (moe_combine_rmsnorm).

- against the oracle: the new residual bit-exact (one rounding of an exact
  sum), the normalised rows within the output tolerance;
- the fused kernel gives the bits of the combine followed by the standalone
  norm (the Fireworks post's trap 2/3: a fusion must not change the norm's
  reduction order);
- a token's rows are the same bits at every T; in-place residual; rows wider
  than the register-held part (D > 8192); T = 0.
"""
import numpy as np
import pytest
import torch

import invariant_moe_amd as moe
import oracle
import synth
from gpu_util import banner, dev, rel_l2, requires_gpu, to_np, tol_for

pytestmark = [pytest.mark.gpu, requires_gpu]

EPS = 1e-6


def _rows(act, seed, tensor, T, D, std=1.0):
    if act == "f32":
        return synth.normal_f32(seed, tensor, T * D, std).reshape(T, D)
    return synth.normal_bf16(seed, tensor, T * D, std).reshape(T, D)


def _gamma(act, seed, D):
    g = np.random.default_rng(seed).uniform(0.5, 2.0, D).astype(np.float32)
    return synth.f32_to_bf16(g) if act == "bf16" else g


def _routing(seed, T, E, k):
    rng = np.random.default_rng(seed)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    w = rng.uniform(0.05, 1.0, (T, k)).astype(np.float32)
    w /= w.sum(1, keepdims=True)
    _, _, _, pair_row = oracle.permute(idx, E)
    return idx, w, pair_row


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 288, 1024, 4096, 7168, 9216])
def test_residual_rmsnorm_vs_oracle(act, D):
    T = 37
    banner(f"residual_rmsnorm act={act} D={D} T={T}")
    x = _rows(act, 81, 0, T, D, 2.0)
    r = _rows(act, 81, 1, T, D, 1.0)
    g = _gamma(act, 82, D)
    h_ref, n_ref = oracle.residual_rmsnorm(x, r, g, EPS)
    h, n = moe.residual_rmsnorm(dev(x), dev(r), dev(g), EPS)
    assert np.array_equal(to_np(h), h_ref)
    rl = rel_l2(to_np(n), n_ref)
    banner(f"normed rel_l2={rl:.3e}")
    assert rl <= tol_for(act), rl
    # in place: residual_out is the residual tensor itself
    rt = dev(r)
    h2, n2 = moe.residual_rmsnorm(dev(x), rt, dev(g), EPS, residual_out=rt)
    assert h2.data_ptr() == rt.data_ptr()
    assert np.array_equal(to_np(rt), h_ref) and np.array_equal(to_np(n2), to_np(n))


@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("k,with_shared", [(8, True), (2, False), (9, True), (32, True)])
def test_combine_rmsnorm_fused_equals_unfused(act, k, with_shared):
    T, E, D = 53, 40, 1056  # 132 chunks: a partial second half of the threads
    banner(f"combine_rmsnorm act={act} k={k} shared={with_shared}")
    idx, w, pair_row = _routing(83, T, E, k)
    o = _rows(act, 84, 0, T * k, D)
    s = _rows(act, 84, 1, T, D) if with_shared else None
    r = _rows(act, 84, 2, T, D)
    g = _gamma(act, 85, D)
    args = (dev(o), dev(idx), dev(w), dev(pair_row), dev(s) if s is not None else None)
    h_f, n_f = moe.combine_rmsnorm(*args, dev(r), dev(g), EPS)
    y = moe.combine(*args)
    h_u, n_u = moe.residual_rmsnorm(y, dev(r), dev(g), EPS)
    assert np.array_equal(to_np(h_f), to_np(h_u))
    assert np.array_equal(to_np(n_f), to_np(n_u))
    h_ref, n_ref = oracle.combine_rmsnorm(o, idx, w, pair_row, s, r, g, EPS, T, k, D)
    assert np.array_equal(to_np(h_f), h_ref)
    rl = rel_l2(to_np(n_f), n_ref)
    banner(f"fused normed rel_l2={rl:.3e}")
    assert rl <= tol_for(act), rl


@pytest.mark.parametrize("fused", [False, True])
def test_tail_rows_equal_at_every_T(fused):
    banner(f"tail batch invariance fused={fused}")
    E, k, D, Tmax = 64, 8, 7168, 1100
    idx, w, pair_row = _routing(86, Tmax, E, k)
    o = _rows("bf16", 87, 0, Tmax * k, D)
    s = _rows("bf16", 87, 1, Tmax, D)
    x = _rows("bf16", 87, 2, Tmax, D)
    r = _rows("bf16", 87, 3, Tmax, D)
    g = dev(_gamma("bf16", 88, D))
    full = None
    for T in (Tmax, 300, 77, 5, 1):
        if fused:
            # the first T tokens: their slots and rows, renumbered
            sub_idx = np.ascontiguousarray(idx[:T])
            _, _, _, sub_pr = oracle.permute(sub_idx, E)
            sub_o = np.empty((T * k, D), np.uint16)
            sub_o[sub_pr] = o[pair_row[:T * k]]
            h, n = moe.combine_rmsnorm(dev(sub_o), dev(sub_idx), dev(np.ascontiguousarray(w[:T])),
                                       dev(sub_pr), dev(np.ascontiguousarray(s[:T])),
                                       dev(np.ascontiguousarray(r[:T])), g, EPS)
        else:
            h, n = moe.residual_rmsnorm(dev(np.ascontiguousarray(x[:T])),
                                        dev(np.ascontiguousarray(r[:T])), g, EPS)
        h, n = to_np(h), to_np(n)
        if full is None:
            full = (h, n)
        else:
            assert np.array_equal(h, full[0][:T]) and np.array_equal(n, full[1][:T]), T


def test_tail_edge_cases():
    banner("tail edge cases")
    D = 64
    g = dev(np.ones(D, np.float32))
    empty = torch.empty((0, D), dtype=torch.float32, device="cuda")
    h, n = moe.residual_rmsnorm(empty, empty, g, EPS)
    assert h.shape == (0, D) and n.shape == (0, D)
    # zero rows stay zero with a positive epsilon; eps must be finite and >= 0
    z = dev(np.zeros((3, D), np.float32))
    _, n = moe.residual_rmsnorm(z, z, g, EPS)
    assert not to_np(n).any()
    for bad in (-1.0, float("inf"), float("nan")):
        with pytest.raises(moe.MoEError):
            moe.residual_rmsnorm(z, z, g, bad)
