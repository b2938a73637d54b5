"""CPU oracle for the minGRU scan, its single-token step and the MinMax scan.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only the test suite, the smoke check and the benchmark's CPU-baseline
leg call it.  It shares no code with the GPU library; the only thing both sides
use is the seeded input generator in ``synth``, which holds no arithmetic of
the method.

Everything here is plain, slow and meant to be checked by eye:

* ``scalar``   -- sigma, softplus, the candidate activation g and log g, fp64.
* ``mingru``   -- the minGRU recurrence run sequentially over t in fp64, the
                  input / output projections, the single-token step, and the
                  two terms of h used to condition the error metric.
* ``logspace`` -- the log-space parallel form (cumulative sum plus a
                  cumulative log-sum-exp), kept as a check that the method's
                  parallel form equals the sequential definition.
* ``minmax``   -- the MinMax neuron's recurrence run sequentially, plus the
                  clamp-composition rule the parallel form relies on.
* ``decay``    -- the minGRU recurrence with per-token time decay of the
                  carried state (gap-driven, clamped), sequentially.
* ``grad``     -- the gradients of both scans (backward in time, chain rule).
* ``metrics``  -- the conditioned error measures used by the parity tests.

Sources: the minGRU-pytorch profile (openvist.com), intro and "Requirements &
limits" (log-space numerically stable version; parallel and sequential modes
with a carried hidden state); the minmaxrnc PyPI page, "The model" item 3 (the
MinMax update) and "Key properties" (bounded operator, prefix-scan depth);
the "Your first delta model" tutorial, Step 5 "Adding time decay" (the decay
contract: a per-event gap decays the carried state at the token boundary).
The pages print no equations for the minGRU layer: the profile names the
layer, its log-space numerically stable evaluation and its two modes.  The
recurrence written out here (h_t = (1 - z_t) h_{t-1} + z_t g(p_t), z =
sigma(k), g(x) = x + 1/2 for x >= 0 else sigma(x), [k, p] = x W_in, with the
log-space coefficients log(1 - z) = -softplus(k) and log z + log g(p)) is the
minGRU recurrence those sections refer to, taken as stated.

Parity status of each function is listed in its module docstring.
"""

from . import decay, grad, logspace, metrics, minmax, mingru, scalar  # noqa: F401
