// Instantiation of the specialised kernels for signature SigL2to3.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL2to3 = make_set<SigL2to3>("L2to3");
}  // namespace e3k
