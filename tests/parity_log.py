"""Record of every tensor that passed the floating-point parity check only through the conditioning
criterion (largest error within K_COND times the oracle's one-ulp perturbation response), so that the
end of a pytest run can list them."""

USES = []


class ConditioningWarning(UserWarning):
    """A tensor missed the elementwise bound and passed on the one-ulp perturbation criterion."""
