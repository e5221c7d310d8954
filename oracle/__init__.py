"""CPU oracle of the KDA recurrence (test infrastructure only).

``kda_oracle`` drives the float64 C implementation, ``kda_np`` is its
independent NumPy twin.  Only tests, the smoke check and the benchmark's CPU
baseline may import this package; the HIP library never does.
"""
