// Kernels of the FP6 e2m3 (1 sign, 2 exponent, 3 mantissa bits) weight format: every
// kernel configuration of the fused linear layer plus the de-quantisation
// export, instantiated for this format (see fpx_device.h).
#include "fpx_device.h"

FPX_DEFINE_FORMAT(e2m3, kE2M3)
