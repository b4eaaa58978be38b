"""Ratios over the R/I/D/A draft counters.

Test infrastructure (see the package docstring).

Definitions (fanout, "Structured output speculative decoding acceptance",
sections "Name the three counters" and "Mean acceptance length uses another
denominator"; infra-guide 5.2, section 7.1):

* R: raw draft tokens the drafter proposed
* I: drafts invalidated by the structured-output constraint
* D = R - I: grammar-eligible drafts
* A: eligible drafts the target verifier accepted
* grammar survival = D / R, conditional acceptance = A / D,
  end-to-end yield = A / R, mean acceptance length = 1 + A / steps
"""


def sd_rates(R, I, A, steps):
    """Return a dict of the three ratios and the mean acceptance length.

    A ratio whose denominator is zero is reported as None.
    """
    R, I, A, steps = int(R), int(I), int(A), int(steps)
    if I > R or A > R - I or min(R, I, A, steps) < 0:
        raise ValueError("counters must satisfy 0 <= A <= R - I, 0 <= I <= R")
    D = R - I
    return {
        "R": R,
        "I": I,
        "D": D,
        "A": A,
        "survival": D / R if R else None,
        "acceptance": A / D if D else None,
        "yield": A / R if R else None,
        "mean_acceptance_length": 1.0 + A / steps if steps else None,
    }
