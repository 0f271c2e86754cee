"""Each plausible mistake planted in the oracle (a dropped diagonal, a sign,
a transposed weight, the flatten order, the gate sign, a missing scale or
normalisation, the wrong key row, an off-by-one decode cache, a chunk that ignores its
cached prefix; in the full layer a missing or misplaced norm, a transposed
projection, a wrong rounding rule) must be caught
by at least one pin.  Mutants are compiled on the CPU into a scratch dir."""
import pytest

import oracle
import pins

MUTANTS = {
    1: "causal mask drops the diagonal",
    2: "softmax exponent sign flipped",
    3: "W_UK read transposed",
    4: "W_UV read transposed",
    5: "value-major flatten of heads",
    6: "sigmoid of the negated gate",
    7: "softmax scale ignored",
    8: "softmax not normalised",
    9: "weighted sum uses the query's own latent row",
    10: "decode drops the newest cached row",
    11: "chunked prefill ignores the cached prefix",
    12: "latent not normalised",
    13: "latent norm gain applied inside the norm",
    14: "query latent not normalised",
    15: "W_q_up read transposed",
    16: "W_gate read transposed",
    17: "W_o read transposed",
    18: "RMSNorm over the sum of squares instead of the mean",
    19: "bf16 rounding ties away from zero",
    20: "paged cache: wrong block-table row stride",
    21: "paged cache: slot within the page off by one",
    22: "backward: softmax Jacobian row term dropped",
    23: "backward: value path of c dropped from dc",
    24: "backward: gate gradient uses the sigmoid, not its derivative",
    25: "backward: query-side gradient missing the softmax scale",
    26: "varlen: the chunk placed at the start of its sequence",
    27: "layer backward: the norm's projection term dropped",
    28: "layer backward: input gradient without the query path",
    29: "kda: decay applied after the write",
    30: "kda: read-out before the write",
    31: "kda: write strength ignored",
    32: "kda: decay sign flipped",
    33: "kda: GVA heads interleaved instead of repeated",
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(mutant, tmp_path):
    o = oracle.build_mutant(mutant, str(tmp_path))
    assert o.mutant == mutant
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passed every pin"
