// hbm_probe.hip -- attainable HBM read rates on this GPU, the measured
// ceilings the QSA kernels are compared with (separate library,
// libhbm_probe.so; not part of the C ABI in include/qsa.h).
//
//   hbm_probe_stream  every byte of a buffer read once, 16 bytes per lane
//                     with four loads in flight per lane (the shape of the
//                     index scan's K_idx stream);
//   hbm_probe_gather  the decode attention's reads without its arithmetic:
//                     for every (problem, chunk, KV head) one wave walks the
//                     chunk's kept cells (ids rows of k cells per problem)
//                     and reads each cell's D int8 K codes, D int8 V codes
//                     and the two D/32 fp16 scale rows of its KV head, at the
//                     same base pointers and byte strides qsa_attend takes,
//                     eight cells per 16-lane group in flight.
// Both fold what they read into one word per workgroup, written to `sink`
// (so nothing is optimised away); the sink contents have no meaning.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void k_probe_stream(const uint4* __restrict__ x, long long n16,
                                                      uint32_t* __restrict__ sink)
{
    uint32_t acc = 0;
    const long long stride = (long long)gridDim.x * 1024;
    for (long long i = (long long)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const long long j = i + 256 * u;
            v[u] = j < n16 ? x[j] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int o = 32; o >= 1; o >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if ((threadIdx.x & 63) == 0)
        atomicXor(sink + blockIdx.x, acc);
}

struct GatherArgs {
    const int8_t* Kq;
    const int8_t* Vq;
    const uint8_t* Ksc;
    const uint8_t* Vsc;
    long long kq_cs, vq_cs, ksc_cs, vsc_cs;  // cell strides, bytes
    long long kq_bs, vq_bs, ksc_bs, vsc_bs;  // batch strides, bytes
    const int32_t* ids;                      // [B][k], values in [0, N)
    int B, k, Hkv, D, chunks;
    uint32_t* sink;
};

// Wave w: problem w / (chunks * Hkv), chunk (w / Hkv) % chunks, KV head
// w % Hkv.  A 16-lane group reads one cell: lane s takes bytes 16 s .. of
// the D-byte code rows (D / 16 <= 16 lanes) and, for s < D / 64, a 4-byte
// word of each scale row.
__global__ __launch_bounds__(256) void k_probe_gather(GatherArgs a)
{
    const long long wave = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int per = a.chunks * a.Hkv;
    if (wave >= (long long)a.B * per)
        return;
    const int b = (int)(wave / per);
    const int g = (int)(wave % a.Hkv), c = (int)((wave / a.Hkv) % a.chunks);
    const int S = (a.k + a.chunks - 1) / a.chunks;
    const int beg = c * S, end = min(beg + S, a.k);
    const int s = lane & 15, cq = lane >> 4;
    const bool code_lane = 16 * s < a.D, scale_lane = 4 * s < a.D / 16;
    const int32_t* idr = a.ids + (size_t)b * a.k;
    const char* kb = (const char*)a.Kq + (long long)b * a.kq_bs + (long long)g * a.D + 16 * s;
    const char* vb = (const char*)a.Vq + (long long)b * a.vq_bs + (long long)g * a.D + 16 * s;
    const char* ksb = (const char*)a.Ksc + (long long)b * a.ksc_bs + (long long)g * (a.D / 16) + 4 * s;
    const char* vsb = (const char*)a.Vsc + (long long)b * a.vsc_bs + (long long)g * (a.D / 16) + 4 * s;
    uint32_t acc = 0;
    for (int t = beg; t < end; t += 32) {
        uint4 kv[8], vv[8];
        uint32_t ks[8], vs[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = idr[min(t + 4 * u + cq, end - 1)];
            kv[u] = code_lane ? *(const uint4*)(kb + j * a.kq_cs) : make_uint4(0u, 0u, 0u, 0u);
            vv[u] = code_lane ? *(const uint4*)(vb + j * a.vq_cs) : make_uint4(0u, 0u, 0u, 0u);
            ks[u] = scale_lane ? *(const uint32_t*)(ksb + j * a.ksc_cs) : 0u;
            vs[u] = scale_lane ? *(const uint32_t*)(vsb + j * a.vsc_cs) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            acc ^= kv[u].x ^ kv[u].y ^ kv[u].z ^ kv[u].w ^ vv[u].x ^ vv[u].y ^ vv[u].z ^
                   vv[u].w ^ ks[u] ^ vs[u];
    }
    for (int o = 32; o >= 1; o >>= 1)
        acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
    if (lane == 0)
        atomicXor(a.sink + blockIdx.x, acc);
}

}  // namespace

extern "C" {

// Reads n_bytes (a multiple of 16, 16-byte aligned x) once with `grid`
// workgroups of 256 threads; sink: at least `grid` uint32 words.  Returns
// the hipError_t of the launch.
__attribute__((visibility("default"))) int hbm_probe_stream(const void* x, long long n_bytes,
                                                            void* sink, int grid, void* stream)
{
    if (!x || !sink || grid < 1 || n_bytes < 0 || n_bytes % 16 || (uintptr_t)x % 16)
        return (int)hipErrorInvalidValue;
    k_probe_stream<<<grid, 256, 0, (hipStream_t)stream>>>((const uint4*)x, n_bytes / 16,
                                                         (uint32_t*)sink);
    return (int)hipGetLastError();
}

// Number of sink words hbm_probe_gather needs.
__attribute__((visibility("default"))) long long hbm_probe_gather_sink_words(int B, int Hkv,
                                                                             int chunks)
{
    return ((long long)B * chunks * Hkv + 3) / 4;
}

// The attention gather of B problems with k kept cells each (ids [B][k]),
// chunks per problem, Hkv heads of D (a multiple of 64 up to 256) codes.
// Pointers and strides as qsa_attend takes them (code rows and bases
// 16-byte aligned, scale rows 4-byte aligned).
__attribute__((visibility("default"))) int hbm_probe_gather(
    const void* Kq, const void* Vq, const void* Ksc, const void* Vsc, long long kq_cs,
    long long vq_cs, long long ksc_cs, long long vsc_cs, long long kq_bs, long long vq_bs,
    long long ksc_bs, long long vsc_bs, const int32_t* ids, int B, int k, int Hkv, int D,
    int chunks, void* sink, void* stream)
{
    if (!Kq || !Vq || !Ksc || !Vsc || !ids || !sink || B < 1 || k < 1 || Hkv < 1 ||
        chunks < 1 || D < 64 || D > 256 || D % 64)
        return (int)hipErrorInvalidValue;
    GatherArgs a{(const int8_t*)Kq, (const int8_t*)Vq, (const uint8_t*)Ksc, (const uint8_t*)Vsc,
                 kq_cs, vq_cs, ksc_cs, vsc_cs, kq_bs, vq_bs, ksc_bs, vsc_bs, ids, B, k, Hkv, D,
                 chunks, (uint32_t*)sink};
    const long long blocks = hbm_probe_gather_sink_words(B, Hkv, chunks);
    k_probe_gather<<<(unsigned)blocks, 256, 0, (hipStream_t)stream>>>(a);
    return (int)hipGetLastError();
}

}  // extern "C"
