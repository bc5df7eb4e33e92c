// Host-emulated build of the scan library (TEST INFRASTRUCTURE): the C-ABI
// source is compiled unchanged against the emulated device header that sits
// next to this file.
#include "../../complex_chunkwise_ssd_amd/csrc/ssd_api.hip"

extern "C" long emu_mfma_count(void) { return emu::g_mfma_count; }

// 0 restores index order; any other value seeds the shuffled thread order.
extern "C" void emu_set_shuffle_seed(unsigned long long seed) { emu::g_shuffle = seed; }

// The kernels' own sin/cos, for an accuracy test against double precision.
extern "C" void emu_sincos(const float *x, float *s, float *c, long n)
{
    for (long i = 0; i < n; ++i)
        ssd::sincos_cw(x[i], &s[i], &c[i]);
}
