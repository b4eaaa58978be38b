"""Plain CPU oracle for the speculative-decoding verifier (rejection sampler).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in the
repository's graft entry module, and the CPU-baseline leg of the benchmark use
it.  It shares no code with the HIP path (no kernels, headers, helpers, tables
or constant generators); the two meet only through the seeded synthetic inputs.

What it computes, and where the pages define it
-----------------------------------------------
* ``verify.sd_verify`` -- standard speculative rejection sampling for a batch
  of requests with k drafted tokens each, in float64 with NumPy:
  grammar bitmask and temperature applied to the target logits, softmax over
  the vocabulary (pyshine "vLLM, part 2", section "Verification: rejection
  sampling on the GPU"), accept with min(1, p/q) and cut at the first rejection
  (vllm-learning "speculative decoding code walkthrough", RejectionSampler),
  resample from max(p - q, 0) or use the argmax rule for temperature zero,
  sample the bonus token after full acceptance, one-hot q for drafts without
  probabilities (infra-guide 5.2, section 4.3), and the R/I/D/A counters
  (fanout "Structured output speculative decoding acceptance", section
  "Name the three counters").
* ``philox`` -- Philox4x32-10 from Salmon, Moraes, Dror and Shaw, "Parallel
  Random Numbers: As Easy as 1, 2, 3" (SC'11), which supplies every uniform
  the sampler draws.  The pages name no generator; this is a reading.
* ``ngram.propose_batch`` / ``ngram.propose_one`` -- the n-gram (prompt lookup)
  draft proposer: the history's tail looked up earlier in the same history,
  longest window first, earliest occurrence on ties, the following tokens
  copied (infra-guide 5.2, sections 4.1 and 6; pyshine "vLLM, part 2",
  "Choosing a drafter").
* ``rates`` -- survival D/R, acceptance A/D, yield A/R and mean acceptance
  length 1 + A/steps (fanout, sections "Work a denominator example" and
  "Mean acceptance length uses another denominator"; infra-guide 5.2 section 7.1).

Pins (tests marked ``not gpu``): the pages' worked counter examples, SciPy's
softmax/logsumexp, NumPy argmax, brute-force top-k, rocRAND's own Philox
compiled on the host, closed forms of the Weyl constants, exact enumeration of
the accept/resample law at V=8, chi-square tests of the sampled tokens, and
for the n-gram proposer the pages' worked lookups, brute force and the
Z-function of the reversed history.
"""

from . import ngram, philox, rates, verify  # noqa: F401
from .verify import sd_verify, sd_verify_ragged  # noqa: F401
from .rates import sd_rates  # noqa: F401
