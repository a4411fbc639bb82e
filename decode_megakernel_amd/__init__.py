"""MI355X-native decode-step megakernel: one persistent HIP launch per decode
step, behind a small C ABI (include/mk.h).  The Python side only marshals
arguments; every step of the decode runs in the HIP kernel."""
