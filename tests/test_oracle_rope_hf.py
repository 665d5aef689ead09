"""Pin of the oracle's RoPE (frequency schedule and pairing) against a library.

The pages fix the pairing only through tiny_agent ``generate.py``,
``_rope_pos`` (halves of the head vector rotated against each other), and
never print the frequencies; the colibri PR "inkling: ring-buffer KV cache"
(section "Tests done") checks its engine against the Hugging Face model.  So
the oracle's ``rope.rotate`` is compared here with ``transformers``' Llama
rotary embedding (``LlamaRotaryEmbedding`` builds the cos/sin tables,
``apply_rotary_pos_emb`` rotates), an implementation that shares nothing with
the oracle.

``transformers`` computes its frequencies and angles in float32 on purpose,
so the comparison cannot be made at float64 precision.  Each check therefore
states the error bound of the library's float32 steps and asserts the
oracle's float64 rotation lies within it:

* frequencies ``1 / base**(2d/D)``: a float32 power (at most 2 ulp) and a
  correctly rounded reciprocal, so a relative error of at most 2**-21;
* angle ``pos * theta``: one more float32 rounding, so
  ``|d angle| <= pos * theta * (2**-21 + 2**-24)``;
* ``cos`` / ``sin`` of a float32 angle: at most 2**-22 absolute;
* the rotation itself runs here in float64 on the upcast tables.

A rotated coordinate mixes two inputs, so its error is at most
``(|x_d| + |x_pair|) * (d angle + 2**-22)``.  With ``base = 2**16`` and
``D = 16`` every frequency is a power of two (``2**(-2d)``) and every angle is
exact in float32, which leaves only the cos/sin rounding: a bound near 1e-6
even at position 32767.

A wrong exponent (``-d/D`` instead of ``-2d/D``) or the interleaved pairing
misses these bounds by orders of magnitude; the mutation tests plant each in
the oracle and require the checks to fail.
"""

import numpy as np
import pytest
import torch

from oracle import rope as orope

transformers = pytest.importorskip("transformers")
from transformers import LlamaConfig  # noqa: E402
from transformers.models.llama.modeling_llama import (  # noqa: E402
    LlamaRotaryEmbedding, apply_rotary_pos_emb)

POSITIONS = np.array([0, 1, 511, 8191, 32767])
FREQ_REL = 2.0 ** -21
TRIG_ABS = 2.0 ** -22


def _hf_rope(head_dim, base):
    cfg = LlamaConfig(hidden_size=head_dim * 4, num_attention_heads=4,
                      num_key_value_heads=2, head_dim=head_dim, rope_theta=float(base),
                      max_position_embeddings=65536)
    return LlamaRotaryEmbedding(cfg)


def _hf_rotate(x, pos, base):
    """x (T, H, D) float64 rotated by transformers at positions pos (T,)."""
    T, H, D = x.shape
    emb = _hf_rope(D, base)
    pid = torch.as_tensor(pos, dtype=torch.int64)[None, :]
    probe = torch.zeros(1, dtype=torch.float32)
    cos, sin = emb(probe, pid)                       # (1, T, D) float32
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]  # (1, H, T, D)
    qr, _ = apply_rotary_pos_emb(xt, xt.clone(), cos.double(), sin.double())
    return qr[0].numpy().transpose(1, 0, 2), emb.inv_freq.double().numpy()


def _bound(x, pos, theta, exact_angles):
    """Per-element bound on |oracle - transformers| for x (T, H, D)."""
    T, H, D = x.shape
    half = D // 2
    pos = np.asarray(pos, dtype=np.float64)
    if exact_angles:
        dang = np.zeros((T, half))
    else:
        dang = pos[:, None] * theta[None, :] * (FREQ_REL + 2.0 ** -24)
    per_pair = (dang + TRIG_ABS)[:, None, :]           # (T, 1, D/2)
    mag = np.abs(x[..., :half]) + np.abs(x[..., half:])
    b = mag * per_pair
    return np.concatenate((b, b), axis=-1) + 1e-15


@pytest.mark.parametrize("head_dim", [64, 128])
def test_rope_frequencies_match_transformers(head_dim):
    # theta_d = base**(-2d/D), d < D/2: transformers' default Llama schedule.
    base = 10000.0
    hf = _hf_rope(head_dim, base).inv_freq.double().numpy()
    ours = orope.inv_freq(head_dim, base)
    assert ours.shape == hf.shape == (head_dim // 2,)
    assert np.all(np.abs(ours - hf) <= FREQ_REL * ours)


@pytest.mark.parametrize("head_dim", [64, 128])
def test_rope_rotation_matches_transformers(head_dim):
    g = np.random.default_rng(head_dim)
    x = g.standard_normal((len(POSITIONS), 3, head_dim))
    base = 10000.0
    ref, _ = _hf_rotate(x, POSITIONS, base)
    got = orope.rotate(x, POSITIONS, base)
    bound = _bound(x, POSITIONS, orope.inv_freq(head_dim, base), exact_angles=False)
    assert np.all(np.abs(got - ref) <= bound)
    # position 0 is the identity on both sides
    assert np.array_equal(got[0], x[0]) and np.abs(ref[0] - x[0]).max() == 0.0


def test_rope_rotation_matches_transformers_exact_angles():
    # base 2**16, D 16: theta_d = 2**(-2d) exactly, so every float32 angle
    # pos * theta_d is exact and only cos / sin rounding separates the two.
    D, base = 16, 65536.0
    theta_hf = _hf_rope(D, base).inv_freq.double().numpy()
    assert np.array_equal(theta_hf, 2.0 ** (-2.0 * np.arange(D // 2)))
    pos = np.concatenate([POSITIONS, [3, 100, 12345, 20000]])
    g = np.random.default_rng(16)
    x = g.standard_normal((len(pos), 2, D))
    ref, _ = _hf_rotate(x, pos, base)
    got = orope.rotate(x, pos, base)
    bound = _bound(x, pos, theta_hf, exact_angles=True)
    assert np.all(np.abs(got - ref) <= bound)
    assert np.abs(got - ref).max() < 2e-6


# ---------------------------------------------------------------------------
# Mutations planted in the oracle: each must fail a check above.
# ---------------------------------------------------------------------------
def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_mutation_rope_exponent_d_over_D(monkeypatch):
    def wrong(head_dim, base):
        d = np.arange(head_dim // 2, dtype=np.float64)
        return np.power(float(base), -d / head_dim)
    monkeypatch.setattr(orope, "inv_freq", wrong)
    assert _fails(test_rope_frequencies_match_transformers, 128)
    assert _fails(test_rope_rotation_matches_transformers, 64)
    assert _fails(test_rope_rotation_matches_transformers_exact_angles)


def test_mutation_rope_interleaved_pairing(monkeypatch):
    def interleaved(x, pos, base):
        x = np.asarray(x, dtype=np.float64)
        ang = orope.angles(pos, x.shape[-1], base)
        c = np.cos(ang)[:, None, :]
        s = np.sin(ang)[:, None, :]
        out = np.empty_like(x)
        out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
        return out
    monkeypatch.setattr(orope, "rotate", interleaved)
    assert _fails(test_rope_rotation_matches_transformers, 128)
    assert _fails(test_rope_rotation_matches_transformers_exact_angles)


def test_mutation_rope_sign_flipped(monkeypatch):
    orig = orope.rotate
    monkeypatch.setattr(orope, "rotate", lambda x, pos, base: orig(x, -np.asarray(pos), base))
    assert _fails(test_rope_rotation_matches_transformers, 64)
