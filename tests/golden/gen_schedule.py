"""Writes schedule.json: closed-form values of the two step schedules the
Colossal-AI distributed-optimizers page prints, evaluated at 30 digits with mpmath.

* beta2t(t) = 1 - t ** decay_rate with decay_rate = -0.8 (note after "Step 5").
* relative step rho(t) = min(1e-2, 1/sqrt(t)); with warmup_init the 1e-2 becomes
  1e-6 * t ("Step 3").

Uses neither the oracle nor the library.
"""
import json
import os

import mpmath as mp

mp.mp.dps = 30
out = {
    "source": "closed forms printed on the Colossal-AI distributed-optimizers page: beta2t = 1 - step**decay_rate (note after 'Step 5'), relative step min(1e-2, 1/sqrt(step)) and its warmup form 1e-6*step ('Step 3')",
    "beta2t": {str(t): float(1 - mp.power(t, mp.mpf("-0.8"))) for t in (1, 2, 3, 4, 10, 100, 40000)},
    "rho": {str(t): float(min(mp.mpf("0.01"), 1 / mp.sqrt(t))) for t in (1, 2, 100, 10000, 40000, 90000)},
    "rho_warmup": {str(t): float(min(mp.mpf("1e-6") * t, 1 / mp.sqrt(t))) for t in (1, 5, 100, 1000)},
}
with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "schedule.json"), "w") as f:
    json.dump(out, f, indent=1)
    f.write("\n")
