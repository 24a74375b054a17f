// MX E2M1 (FP4) levels 5-6 and the MX dispatch over element formats.
#include "kernels_fast.hpp"

namespace mce {

// FP4: gemm_early in byte units, with whole scale groups (K a multiple of
// 512 elements, 16-byte scale rows) and 16-byte aligned rows.
hipError_t launch_fast_fp4(int level, const GemmArgs &p, hipStream_t s)
{
    if (p.K % 512 != 0 || p.lda % 32 != 0 || p.ldb % 32 != 0 || p.ld_sa % 16 != 0 ||
        p.ld_sb % 16 != 0 || (uintptr_t)p.SA % 16 != 0 || (uintptr_t)p.SB % 16 != 0)
        return hipErrorInvalidValue;
    GemmArgs q = p;
    q.K = p.K / 2;
    q.lda = p.lda / 2;
    q.ldb = p.ldb / 2;
    switch (level) {
    case 5: return launch_early<Fp4Ring128G, 256, 256, false>(q, s);
    case 6: return launch_early<Fp4Ring128G, 256, 256, true>(q, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fast_mx(int level, const GemmArgs &p, hipStream_t s)
{
    if (mx_bits(p.mx_fmt) == 8 && (p.a_cm != 0 || p.b_cm == 0))
        return launch_fast_mx_mn(level, p, s);
    switch (p.mx_fmt) {
    case MX_E2M1: return launch_fast_fp4(level, p, s);
    case MX_E4M3: return launch_fast_e4m3(level, p, s);
    case MX_E5M2: return launch_fast_e5m2(level, p, s);
    case MX_E2M3: case MX_E3M2: return launch_fast_fp6(level, p, s);
    default: return hipErrorInvalidValue;
    }
}

} // namespace mce
