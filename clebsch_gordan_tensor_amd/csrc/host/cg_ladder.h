// Host-side Clebsch-Gordan generator for the HIP library.
//
// Builds the real-basis coupling blocks T^{(l1,l2,L)}[M][m1][m2] by the
// construction of the e3j paper, Appendix G.2 (Eq.22-25): the top state
// |L L> of V_l1 (x) V_l2 solves the J^2 eigen-equation restricted to total
// spin M = L, a three-term recurrence that is solved as a triangular system;
// the lower states follow by applying J_- = J_-^(1) + J_-^(2) (the Leibniz
// rule of G.2) and renormalising.  Phase: the top state has a positive
// component on m1 = l1 (Condon-Shortley).  The complex blocks are then moved
// to the real harmonic basis (m = -l..l, component-normalised harmonics)
// and kept as their real part (l1+l2+L even) or imaginary part (odd).
#pragma once

#include <vector>

namespace e3 {

// Complex-basis block C[M][m1][m2] = <l1 m1 l2 m2 | L M> (indices shifted by
// +l), all real.  Returns false if the triple does not couple.
bool cg_complex_block(int l1, int l2, int L, std::vector<double>& out);

// Real-basis block T[M][m1][m2] (indices shifted by +l).
bool cg_real_block(int l1, int l2, int L, std::vector<double>& out);

}  // namespace e3
