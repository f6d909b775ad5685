"""CPU oracle of the FLUX.3 Image Klein denoiser.  Test infrastructure only:
imported by tests/, by the package smoke check and by the bench's CPU-baseline
leg, never by the HIP library."""
from .flux3_oracle import *  # noqa: F401,F403
