// The dropout instances of the one-wave dK/dV pass, built with the compiler's default
// choice of accumulation registers (fa_bwd_rk.hip holds the kernel and says why its other
// instances are built differently).
#define FA_RK_DROPOUT 1
#include "fa_bwd_rk.hip"
