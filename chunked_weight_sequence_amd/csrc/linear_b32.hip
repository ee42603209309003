// The b = 32 TTT-Linear kernels in a translation unit of their own, so that they can be compiled
// with a different instruction scheduler from the rest of linear.hip (see build.py).
#define TTT_LINEAR_B32_TU 1
#include "linear.hip"
