// Kernels of the FP6 e3m2 (1 sign, 3 exponent, 2 mantissa bits) weight format: every
// kernel configuration of the fused linear layer plus the de-quantisation
// export, instantiated for this format (see fpx_device.h).
#include "fpx_device.h"

FPX_DEFINE_FORMAT(e3m2, kE3M2)
