// Instantiation of the specialised kernels for signature SigL1.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL1 = make_set<SigL1>("L1");
}  // namespace e3k
