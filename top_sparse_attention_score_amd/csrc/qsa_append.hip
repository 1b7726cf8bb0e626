// qsa_append.hip -- the KV append kernel (device code in qsa_append.h) and
// its launcher.
#include "qsa_append.h"

namespace qsa {

__global__ __launch_bounds__(256) void k_kv_append(AppendLaunch a, long long q_lanes,
                                                   long long n_quant, long long n_idx)
{
    append_blocks(a, q_lanes, n_quant, n_idx, blockIdx.x, gridDim.x);
}

hipError_t launch_kv_append(const AppendLaunch& a, hipStream_t s)
{
    // Quantisation lanes rounded up to whole workgroups, so no workgroup
    // mixes the two kinds of items (the extra lanes are idle).
    const long long q_lanes = (long long)a.B * a.T * a.Hkv * (a.D / 32) * 2 * 8;
    const long long n_quant = (q_lanes + 255) / 256 * 256;
    const long long n_idx = a.kidx_new ? (long long)a.B * a.T * (a.DI / 4) : 0;
    const long long blocks = (n_quant + n_idx + 255) / 256;
    k_kv_append<<<(unsigned)(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(a, q_lanes, n_quant,
                                                                          n_idx);
    return hipGetLastError();
}

}  // namespace qsa
