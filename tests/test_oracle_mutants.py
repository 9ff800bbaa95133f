"""Planted-mistake checks: each plausible slip in the oracle (a transposed
operand, a wrong axis, a flipped sign, a wrong bit order, a missing
normalization, an off-by-one group) is planted in a copy of one oracle
function on the CPU, and at least one pin of ``test_oracle_pins`` must then
fail.  This shows the pins are strong enough to catch it.  No GPU.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.vq as vq
from tests import test_oracle_pins as pins

# pins run against each mutant (name, callable)
PIN_CALLS = [
    ("hand_vectors", pins.test_pack_hand_vectors),
    ("bit_positions", pins.test_pack_bit_positions_by_definition),
    ("hand_vq", pins.test_hand_worked_vq_example),
    ("oc_scalar", pins.test_oc_entries_by_scalar_loop),
    ("bruteforce_4_3", lambda: pins.test_gemv_equals_bruteforce_dequant(16, 5, 4, 3, 1)),
    ("bruteforce_8_4", lambda: pins.test_gemv_equals_bruteforce_dequant(32, 9, 8, 4, 2)),
    ("bruteforce_4_8", lambda: pins.test_gemv_equals_bruteforce_dequant(64, 16, 4, 8, 1)),
    ("exhaustive", pins.test_exhaustive_two_subvectors_two_bits),
    ("one_hot", pins.test_one_hot_input_reads_a_weight_column),
    ("walsh", pins.test_hadamard_matches_walsh_definition),
    ("h4", pins.test_hadamard_textbook_h4),
    ("orth_64", lambda: pins.test_hadamard_orthogonal(64)),
    ("rht_hand", pins.test_rht_hand_worked_and_norm),
    ("rht_onehot", pins.test_rht_one_hot_and_involution),
    ("res_hand", pins.test_residual_hand_worked),
    ("res_bf", pins.test_residual_bruteforce_dense),
    ("res_ones", pins.test_residual_all_ones_closed_form),
    ("composed", pins.test_gemv_residual_composes_parts),
]


def _oc_strided(x, wc, d):
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B, K = xf.shape
    X = xf.reshape(B, d, K // d).transpose(0, 2, 1)      # wrong subvector axis
    return X @ np.asarray(wc, dtype=np.float64).T


def _oc_wc_reversed(x, wc, d):
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B, K = xf.shape
    w = np.asarray(wc, dtype=np.float64)[:, ::-1]       # centroid components reversed
    return xf.reshape(B, K // d, d) @ w.T


def _lookup_shifted(oc, idx):
    B, J, _ = oc.shape
    ii = np.asarray(idx, dtype=np.int64)
    jj = (np.arange(J)[None, :] + 1) % J                 # subvector off by one
    return np.stack([oc[b][jj, ii].sum(axis=1) for b in range(B)])


def _lookup_dropped_term(oc, idx):
    B, J, _ = oc.shape
    ii = np.asarray(idx, dtype=np.int64)
    jj = np.arange(J)[None, :]
    return np.stack([oc[b][jj, ii][:, 1:].sum(axis=1) for b in range(B)])


def _pack_msb_first(values, nbits):
    v = np.asarray(values, dtype=np.int64).reshape(-1)
    bits = ((v[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.uint8)
    return np.packbits(bits.reshape(-1), bitorder="big")


def _unpack_msb_first(packed, count, nbits):
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    bits = np.unpackbits(p, bitorder="big")[: count * nbits].reshape(count, nbits)
    return (bits.astype(np.int64) << np.arange(nbits)[None, :]).sum(axis=1)


def _hadamard_wrong_sign(h):
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < h:
        H = np.block([[H, -H], [H, H]])
    return H


def _rht_unnormalized(x, sign, had_block):
    return vq.rht.__wrapped_original__(x, sign, had_block) * math.sqrt(had_block)


def _rht_sign_after(x, sign, had_block):
    xf = np.atleast_2d(np.asarray(x, dtype=np.float64))
    B, K = xf.shape
    h = had_block
    H = vq.sylvester_hadamard(h).astype(np.float64)
    out = np.einsum("pq,bnq->bnp", H, xf.reshape(B, K // h, h)).reshape(B, K)
    return out * np.asarray(sign, dtype=np.float64)[None, :] / math.sqrt(h)


def _residual_flipped(x_rot, signs_packed, alpha, N, K, group):
    return -vq.residual_term.__wrapped_original__(x_rot, signs_packed, alpha, N, K, group)


def _residual_group_shift(x_rot, signs_packed, alpha, N, K, group):
    a = np.roll(np.asarray(alpha, dtype=np.float64).reshape(N, K // group), 1, axis=1)
    return vq.residual_term.__wrapped_original__(x_rot, signs_packed, a, N, K, group)


MUTANTS = {
    "oc_strided_subvectors": ("output_codebook", _oc_strided),
    "oc_reversed_centroid": ("output_codebook", _oc_wc_reversed),
    "lookup_off_by_one": ("lookup_sum", _lookup_shifted),
    "lookup_dropped_term": ("lookup_sum", _lookup_dropped_term),
    "pack_msb_first": ("pack_bits", _pack_msb_first),
    "unpack_msb_first": ("unpack_bits", _unpack_msb_first),
    "hadamard_wrong_sign": ("sylvester_hadamard", _hadamard_wrong_sign),
    "rht_unnormalized": ("rht", _rht_unnormalized),
    "rht_sign_after_transform": ("rht", _rht_sign_after),
    "residual_sign_flipped": ("residual_term", _residual_flipped),
    "residual_group_shift": ("residual_term", _residual_group_shift),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    fname, fn = MUTANTS[mutant]
    original = getattr(vq, fname)
    fn.__wrapped_original__ = original
    monkeypatch.setattr(vq, fname, fn)
    monkeypatch.setattr(oracle, fname, fn)
    failed = []
    for name, call in PIN_CALLS:
        try:
            call()
        except Exception:            # AssertionError or a shape error
            failed.append(name)
    assert failed, f"no pin caught mutant {mutant}"


def test_unmutated_oracle_passes_every_pin():
    for name, call in PIN_CALLS:
        call()
