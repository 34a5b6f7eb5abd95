// One-token recurrent update with readout, for generation, on gfx950: per lane
// E <- s E + B (B = v direct, (1 - s) v controlled), evaluated as the scans' step (update()),
// then y = q E / sqrt(mean_h E^2 + eps).
// Page "Entangled State Attention", section "[ ARCHITECTURE ]" (one-token update reusing the
// state) and "[ QUICK START ]" (decode_step); page "Entangled State Attention v2.1",
// section 5 (lightning_step).  The fp32 state is updated in place.
//
// Also the small utility kernels of the library: a zero fill (used instead of
// hipMemsetAsync so that callers may capture the library's work in a graph), an fp32 fill
// and copy (states of an empty sequence), and the composition of sequence-segment
// aggregates.
#include "esa_common.hpp"

namespace esa {

template <typename T, int MODE, int DH, int NT>
__global__ __launch_bounds__(NT) void step_kernel(StepParams p) {
    constexpr int VEC = Storage<T>::VEC;
    constexpr int HL = DH / VEC;
    constexpr int ES = sizeof(T);
    const int64_t lane0 = ((int64_t)blockIdx.x * NT + threadIdx.x) * VEC;
    const bool ok = lane0 < p.nLanes;  // a head is all in or all out: nLanes % DH == 0
    float st[VEC], av[VEC], vv[VEC], qv[VEC];
    uint4 ra = make_uint4(0, 0, 0, 0), rv = ra, rq = ra;
#pragma unroll
    for (int e = 0; e < VEC; ++e) st[e] = 0.0f;
    if (ok) {
        ra = ld16<T>(p.a, lane0, ES);
        rv = ld16<T>(p.v, lane0, ES);
        rq = ld16<T>(p.q, lane0, ES);
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            const float4 x = *reinterpret_cast<const float4*>(p.state + lane0 + e);
            st[e] = x.x;
            st[e + 1] = x.y;
            st[e + 2] = x.z;
            st[e + 3] = x.w;
        }
    }
    unpack<T>(ra, av);
    unpack<T>(rv, vv);
    unpack<T>(rq, qv);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float u = gate_u(av[e]);
        st[e] = update<float>(st[e], 1.0f - u, step_b<MODE, float>(u, vv[e]));
        ss += st[e] * st[e];
    }
    ss = head_sum<HL>(ss);
    const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DH) + kEps);
    float yv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) yv[e] = qv[e] * (st[e] * r);
    if (ok) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
            *reinterpret_cast<float4*>(p.state + lane0 + e) =
                make_float4(st[e], st[e + 1], st[e + 2], st[e + 3]);
        st16<T>(p.y, lane0, ES, pack<T>(yv));
    }
}

template <typename T, int MODE, int DH>
hipError_t launch_step(const StepParams& p, hipStream_t s) {
    // small workgroups: a decode step has few lanes (B*H*Dh / VEC threads), and one wave per
    // workgroup spreads them over more CUs, which shortens the step (launch-latency-bound)
    constexpr int NT = 64;
    constexpr int VEC = Storage<T>::VEC;
    const int64_t threads = (p.nLanes + VEC - 1) / VEC;
    const int64_t blocks = (threads + NT - 1) / NT;
    hipLaunchKernelGGL((step_kernel<T, MODE, DH, NT>), dim3((uint32_t)blocks), dim3(NT), 0, s, p);
    return hipGetLastError();
}

#define ESA_INST_STEP(T, M, D) template hipError_t launch_step<T, M, D>(const StepParams&, hipStream_t);
#define ESA_INST_STEP_D(T, M) \
    ESA_INST_STEP(T, M, 16) ESA_INST_STEP(T, M, 32) ESA_INST_STEP(T, M, 64) ESA_INST_STEP(T, M, 128)
ESA_INST_STEP_D(float, 0)
ESA_INST_STEP_D(float, 1)
ESA_INST_STEP_D(_Float16, 0)
ESA_INST_STEP_D(_Float16, 1)
ESA_INST_STEP_D(__bf16, 0)
ESA_INST_STEP_D(__bf16, 1)
ESA_INST_STEP_D(f8e4m3, 0)
ESA_INST_STEP_D(f8e4m3, 1)
ESA_INST_STEP_D(f8e5m2, 0)
ESA_INST_STEP_D(f8e5m2, 1)

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* dst, int64_t nwords, uint8_t* tail,
                                                        int64_t ntail) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) dst[i] = 0u;
    if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s) {
    if (bytes == 0) return hipSuccess;
    // the workspace pointer is 16-byte aligned (checked by the caller): words, then the tail
    const int64_t nwords = (int64_t)(bytes / 4);
    const int64_t ntail = (int64_t)(bytes - (size_t)nwords * 4);
    int64_t blocks = (nwords + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(dst), nwords, static_cast<uint8_t*>(dst) + nwords * 4,
                       ntail);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy_f32_kernel(float* dst, const float* src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.0f;
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* dst, float value, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = value;
}

hipError_t launch_fill_f32(float* dst, float value, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_f32_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, dst, value, n);
    return hipGetLastError();
}

// Advances the workspace's device epoch (bit 29 set, 29 bits of count) for the scan launch
// recorded after it in the same graph.
__global__ __launch_bounds__(64) void epoch_bump_kernel(uint32_t* word) {
    if (threadIdx.x == 0) {
        const uint32_t e = *word;
        *word = ((e + 1u) & kHostEpochMask) | kDeviceEpochBit;
    }
}

hipError_t launch_epoch_bump(uint32_t* word, hipStream_t s) {
    hipLaunchKernelGGL(epoch_bump_kernel, dim3(1), dim3(64), 0, s, word);
    return hipGetLastError();
}

// Composition of sequence-segment aggregates, per lane, in segment order (forward) or from
// the last segment (reverse): the pair combine (P, E) o c = P c + E of the scan, applied to
// the boundary value segment after segment.  carry[k] receives the value entering segment k
// from its earlier side (forward: the state at its start; reverse: the gradient at its end);
// total receives the value after the last one.
__global__ __launch_bounds__(256) void compose_kernel(int64_t nseg, int64_t nLanes, int reverse,
                                                      const float* prod, const float* agg,
                                                      const float* boundary, float* carry,
                                                      float* total) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < nLanes; l += stride) {
        float c = boundary ? boundary[l] : 0.0f;
        for (int64_t q = 0; q < nseg; ++q) {
            const int64_t k = reverse ? nseg - 1 - q : q;
            carry[k * nLanes + l] = c;
            c = prod[k * nLanes + l] * c + agg[k * nLanes + l];
        }
        if (total) total[l] = c;
    }
}

hipError_t launch_compose(int64_t nseg, int64_t nLanes, int reverse, const float* prod,
                          const float* agg, const float* boundary, float* carry, float* total,
                          hipStream_t s) {
    int64_t blocks = (nLanes + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(compose_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, nseg, nLanes,
                       reverse, prod, agg, boundary, carry, total);
    return hipGetLastError();
}

hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_f32_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, dst, src, n);
    return hipGetLastError();
}

}  // namespace esa
