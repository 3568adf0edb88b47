// Instantiation of the specialised kernels for signature SigL1to3.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL1to3 = make_set<SigL1to3>("L1to3");
}  // namespace e3k
