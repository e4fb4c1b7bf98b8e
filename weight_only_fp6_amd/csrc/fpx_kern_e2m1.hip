// Kernels of the FP4 e2m1 (1 sign, 2 exponent, 1 mantissa bit) weight format: every
// kernel configuration of the fused linear layer plus the de-quantisation
// export, instantiated for this format (see fpx_device.h).
#include "fpx_device.h"

FPX_DEFINE_FORMAT(e2m1, kE2M1)
