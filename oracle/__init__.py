"""fp64 CPU oracle for the gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``, never by the product path.  It shares no code with the
HIP library or its binding.

Parity pins (see ``tests/test_oracle_pins.py``): brute-force causal linear attention, the
gated-linear-attention closed form, exact memory with unit keys, the per-step key-readback
identity, a hand-worked 2x2 example, the explicit matrix forms of the scalar, KDA and
FG2-GDN updates, the gradient-step reading of the delta rule, linearity, state resume, the
norm bound and the dk = dv = 1 closed form; for packed sequences, equality with the dense
batch at equal lengths, isolation between sequences, empty sequences, split invariance (the
prefill-to-decode handoff) and the one-token closed form; for FG2's per-channel rate, its
explicit matrix form, the KDA form at a channel-constant rate, and the gradient-step reading
with a diagonal learning-rate matrix; for the gradients (recurrence_bwd), central finite
differences of the forward along random directions and torch autograd through a separately
written torch forward.  No function here is "parity unpinned".
"""
from .recurrence import (as_f64, decode_step, recurrence, recurrence_bwd, recurrence_fg2, recurrence_fg2_bwd,
                         recurrence_varlen)

__all__ = ["recurrence", "recurrence_bwd", "recurrence_fg2", "recurrence_fg2_bwd", "recurrence_varlen",
           "decode_step", "as_f64"]
