"""Per-sequence status bits reported by the verify and commit steps.

The walkthrough's 5.1 asks an implementation to check numerical validity
under finite precision without fixing a rule; the Atlas lesson states that a
token with q(x) = 0 cannot be proposed and that the residual is used only when
its mass is positive.  These bits record where an input broke those
assumptions; the call itself never fails on them.
"""
ST_DRAFT_OOR = 1     # a draft id lies outside [0, V): treated as a mismatch / rejection
ST_Q_ZERO = 2        # q(x) == 0 at a proposed x: acceptance 1 if p(x) > 0, else 0
ST_RESID_ZERO = 4    # the row to draw from had no positive mass (fallback used)
ST_NONFINITE = 8     # a gathered probability or a drawn row's mass is not finite
ST_BAD_STATE = 16    # commit: n_b outside [0, E] or e_b outside [0, k+1]
ST_CAPACITY = 32     # commit: E < 0 or E + k + 1 > C
