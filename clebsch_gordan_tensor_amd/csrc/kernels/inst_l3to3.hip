// Instantiation of the specialised kernels for signature SigL3to3.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL3to3 = make_set<SigL3to3>("L3to3");
}  // namespace e3k
