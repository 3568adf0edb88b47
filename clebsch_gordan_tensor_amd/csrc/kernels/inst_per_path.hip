// Instantiation of the specialised kernels with one output block per path
// (e3j's default output layout) for signatures SigL1, SigL1to3, SigL2to3.
#include "conv_kernels.h"
#include "signatures.h"

namespace e3k {
const KernelSet kSetL1PP = make_set<PerPath<SigL1>>("L1/per-path");
const KernelSet kSetL1to3PP = make_set<PerPath<SigL1to3>>("L1to3/per-path");
const KernelSet kSetL2to3PP = make_set<PerPath<SigL2to3>>("L2to3/per-path");
}  // namespace e3k
