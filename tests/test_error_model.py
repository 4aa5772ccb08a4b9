"""The per-row LSE and per-slot mass bars (tests/error_model.py) on the CPU.

Two things are checked against the oracle, with no GPU:
  * the bars cover the roundings the kernels perform: an emulation that rounds
    the rotated queries and keys and the probabilities to bf16 the way the
    kernels do, then computes in float64, stays inside them;
  * they discriminate: a 2e-3 offset planted in the oracle's LSE and a 0.5%
    scale planted in its mass both fail them on the Llama-like layer and on a
    small long-context shape.
"""
import numpy as np
import pytest

import oracle
from position_independent_attention_amd import workloads as W
from tests import error_model as E
from tests.util import LSE_ABS, MASS_FLOOR, MASS_REL, lse_bar, lse_errors, mass_bar

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _round_bf16(x):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.asarray(x, np.float32))).astype(np.float64)


def _emulate(w):
    """LSE [total_q, Hq] and mass [B, stride] computed in float64 from bf16
    roundings of the rotated operands and of the probabilities (the kernels'
    rounding points), with the query rows' LSE taken from the emulation."""
    d, G = w.head_dim, w.num_q_heads // w.num_kv_heads
    lse = np.full((w.total_q, w.num_q_heads), -np.inf)
    mass = np.zeros(w.kv_pos.shape)
    q_all = W.bf16_bits_to_f32(w.q).astype(np.float64)
    for r in range(w.batch):
        q0, q1 = int(w.q_start[r]), int(w.q_start[r + 1])
        slots, pis, blks = E._usable_slots(w, r)
        for g in range(w.num_kv_heads):
            kr = _round_bf16(E._keys(w, r, g, slots, pis, blks))
            tt = np.repeat(np.arange(q0, q1), G)
            hh = np.tile(np.arange(g * G, (g + 1) * G), q1 - q0)
            pos = w.q_pos[tt].astype(np.int64)
            qr = _round_bf16(E._rotate(q_all[tt, hh], pos, w.rope_theta))
            vis = pis[None, :] <= pos[:, None]
            s = np.where(vis, qr @ kr.T / np.sqrt(d), -np.inf)
            m = s.max(axis=1)
            p = _round_bf16(np.where(vis, np.exp(s - m[:, None]), 0.0))
            ls = m + np.log(p.sum(axis=1))
            lse[tt, hh] = ls
            # the mass pass rounds its own scaled query and the probability
            qm = _round_bf16(qr / np.sqrt(d) * np.log2(np.e)) / np.log2(np.e)
            sm = np.where(vis, qm @ kr.T, -np.inf)
            mass[r, slots] += _round_bf16(np.exp(sm - ls[:, None])).sum(axis=0)
    return lse, mass


@pytest.mark.parametrize("name", ["tiny", "llama_layer", "long_context_small", "gqa8_short"])
def test_bars_cover_the_kernels_roundings(name):
    w = {"tiny": W.tiny, "llama_layer": W.llama_layer,
         "long_context_small": lambda: W.long_context(n_spans=4, span_tok=512, q_len=64),
         "gqa8_short": lambda: W.custom(130, Hq=16, Hkv=2, d=128, theta=5e5, span_lens=[[40, 9]],
                                        q_len=[21])}[name]()
    ref_o, ref_l = oracle.attention(w)
    ref_m = oracle.mass(w)
    em_l, em_m = _emulate(w)
    mx, ratio = lse_errors(w, em_l, ref_l)
    assert ratio <= 0.7, (name, mx, ratio)
    bar = mass_bar(w, ref_m)
    for r in range(w.batch):
        n = int(w.kv_len[r])
        assert np.all(np.abs(em_m[r, :n] - ref_m[r, :n]) <= 0.7 * bar[r, :n]), r


@pytest.mark.parametrize("name", ["llama_layer", "long_context_small"])
def test_planted_lse_offset_and_mass_scale_fail_the_bars(name):
    w = W.llama_layer() if name == "llama_layer" else W.long_context(n_spans=4, span_tok=512, q_len=64)
    _, ref_l = oracle.attention(w)
    ref_m = oracle.mass(w)
    # the oracle against itself passes
    assert lse_errors(w, ref_l, ref_l)[1] == 0.0
    _, ratio = lse_errors(w, ref_l + 2e-3, ref_l)
    assert ratio > 1.0, ratio
    # the old uniform cap would have let the offset through
    assert 2e-3 <= LSE_ABS
    bar = mass_bar(w, ref_m)
    n = int(w.kv_len[0])
    planted = ref_m[0, :n] * 1.005
    assert np.any(np.abs(planted - ref_m[0, :n]) > bar[0, :n])
    # ... and so would the uniform mass cap
    assert np.all(np.abs(planted - ref_m[0, :n]) <= MASS_REL * ref_m[0, :n] + MASS_FLOOR)


def test_bars_are_capped_and_grow_for_short_rows():
    w = W.custom(131, Hq=4, Hkv=1, d=64, theta=1e4, span_lens=[[3], [900]], q_len=[2, 2])
    b = lse_bar(w)
    assert np.all(b <= LSE_ABS)
    # the request with 5 visible keys gets a wider bar than the one with ~900
    assert b[:2].min() > b[2:].max()
