// Ring-kernel instances with 192-column block tiles (see gemm_w4_ring_impl.h).
#define FCW4_RING_BN 192
#include "gemm_w4_ring_impl.h"
