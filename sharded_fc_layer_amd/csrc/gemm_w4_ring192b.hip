// Ring-kernel instances with 192-column block tiles and two A and three B
// LDS tiles (see gemm_w4_ring_impl.h).
#define FCW4_RING_BN 192
#define FCW4_RING_NA 2
#include "gemm_w4_ring_impl.h"
