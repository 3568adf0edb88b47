// Instantiation of the specialised kernels for signature SigL1to3All.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL1to3All = make_set<SigL1to3All>("L1to3all");
}  // namespace e3k
