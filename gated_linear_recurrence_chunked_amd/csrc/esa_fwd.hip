// Forward scan of the ESA gated linear recurrence with fused gate and per-head RMSNorm
// readout, for gfx950.  One pass over HBM: a, v, q are read once and y is written once.
//
// Recurrence and gates: page "entangled-state-attention 0.1.0", section "Core idea" (direct
// and controlled ESA); readout y = q * Norm(E_t) from the same section, with Norm read as
// per-head RMSNorm (eps 1e-6, no gain); composition over the sequence and the compact final
// state: page "Entangled State Attention", section "[ ARCHITECTURE ]".
#include "esa_common.hpp"

namespace esa {

template <typename T, int MODE, int DH, int L, int NT>
__global__ __launch_bounds__(NT) void fwd_kernel(FwdParams p) {
    using G = Geom<T, DH, L, NT>;
    constexpr int VEC = G::VEC, CB = G::CB, NCL = G::NCL, S = G::S, HL = G::HL;
    constexpr int TT = G::TT;
    constexpr int ES = sizeof(T);

    __shared__ float sP[S][CB];
    __shared__ float sE[S][CB];
    __shared__ float sCarry[CB];

    const uint32_t wg = blockIdx.x;
    const uint32_t tile = wg / p.nCB;
    const uint32_t cb = wg - tile * p.nCB;
    const uint32_t tagAgg = make_tag(p.epoch, kTagAgg);
    const uint32_t tagInc = make_tag(p.epoch, kTagInc);
    const bool readout = p.y != nullptr;

    const int tid = threadIdx.x;
    const int j = tid % NCL;
    const int slot = tid / NCL;
    const int64_t lane0 = (int64_t)cb * CB + j * VEC;  // first flattened (b, h, d) lane
    const bool lane_ok = lane0 < p.nLanes;
    const int64_t b = lane_ok ? lane0 / p.C : 0;
    const int64_t c = lane_ok ? lane0 - b * p.C : 0;
    const int64_t t0 = (int64_t)tile * TT + (int64_t)slot * L;
    const int64_t base = (b * p.T + t0) * p.C + c;

    // ---- load the thread's L steps (all loads issued before any use) ----
    uint4 ra[L], rv[L], rq[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        ra[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
        rq[i] = make_uint4(0, 0, 0, 0);
        if (lane_ok && t0 + i < p.T) {
            ra[i] = ld16(p.a, base + i * p.C, ES);
            rv[i] = ld16(p.v, base + i * p.C, ES);
            if (readout) rq[i] = ld16(p.q, base + i * p.C, ES);
        }
    }

    // ---- level 1: gates and the thread's own fold ----
    float A[L][VEC], Bt[L][VEC];
    float P[VEC], E[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        P[e] = 1.0f;
        E[e] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = lane_ok && t0 + i < p.T;
        float av[VEC], vv[VEC];
        unpack<T>(ra[i], av);
        unpack<T>(rv[i], vv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float s, u;
            gate(av[e], s, u);
            A[i][e] = ok ? s : 1.0f;
            Bt[i][e] = ok ? (MODE == kDirect ? vv[e] : u * vv[e]) : 0.0f;
            E[e] = A[i][e] * E[e] + Bt[i][e];
            P[e] = P[e] * A[i][e];
        }
    }

    // ---- level 2: slot pairs through LDS, scanned in order by wave 0 ----
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        sP[slot][j * VEC + e] = P[e];
        sE[slot][j * VEC + e] = E[e];
    }
    __syncthreads();

    if (tid < kWave) {
#pragma unroll
        for (int k = 0; k < G::CPL; ++k) {
            const int ch = tid + k * kWave;
            float tp = 1.0f, te = 0.0f;
#pragma unroll 8
            for (int s = 0; s < S; ++s) {
                const float ps = sP[s][ch], es = sE[s][ch];
                sP[s][ch] = tp;  // exclusive prefix of slot s within the tile
                sE[s][ch] = te;
                te = ps * te + es;
                tp = tp * ps;
            }
            // ---- level 3: decoupled look-back across tiles ----
            const int64_t gl = (int64_t)cb * CB + ch;
            float carry = 0.0f;
            if (gl < p.nLanes) {
                uint64_t* X = p.flagX + (int64_t)tile * p.nLanes + gl;
                if (tile == 0) {
                    carry = p.e0 ? p.e0[gl] : 0.0f;
                } else {
                    publish(X, tagAgg, te);
                    publish(p.flagY + (int64_t)tile * p.nLanes + gl, tagAgg, tp);
                    carry = look_back(p.flagX, p.flagY, p.nLanes, gl, tile, -1, tagAgg, tagInc, p.hdr);
                }
                publish(X, tagInc, te + tp * carry);
            }
            sCarry[ch] = carry;
        }
    }
    __syncthreads();

    // ---- carry in, re-run the recurrence, readout ----
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const int ch = j * VEC + e;
        E[e] = sE[slot][ch] + sP[slot][ch] * sCarry[ch];
    }
    const int64_t ckbase = b * p.nck;
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t t = t0 + i;
        const bool ok = lane_ok && t < p.T;
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            E[e] = A[i][e] * E[e] + Bt[i][e];
            ss += E[e] * E[e];
        }
        if (readout) {
            ss = head_sum<HL>(ss);
            const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DH) + kEps);
            float qv[VEC], yv[VEC];
            unpack<T>(rq[i], qv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) yv[e] = qv[e] * (E[e] * r);
            if (ok) st16(p.y, base + i * p.C, ES, pack<T>(yv));
        }
        if (ok && p.ckpt && (((t + 1) % kCkptChunk) == 0 || t == p.T - 1)) {
            float* dst = p.ckpt + (ckbase + t / kCkptChunk) * p.C + c;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(E[e], E[e + 1], E[e + 2], E[e + 3]);
        }
        if (ok && p.eT && t == p.T - 1) {
            float* dst = p.eT + lane0;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(E[e], E[e + 1], E[e + 2], E[e + 3]);
        }
    }
}

template <typename T, int MODE, int DH>
hipError_t launch_fwd(const FwdParams& p, hipStream_t s) {
    using C = FwdCfg<T, DH>;
    hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT>), dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
    return hipGetLastError();
}

#define ESA_INST_FWD(T, M, D) template hipError_t launch_fwd<T, M, D>(const FwdParams&, hipStream_t);
#define ESA_INST_FWD_D(T, M) \
    ESA_INST_FWD(T, M, 16) ESA_INST_FWD(T, M, 32) ESA_INST_FWD(T, M, 64) ESA_INST_FWD(T, M, 128)
ESA_INST_FWD_D(float, 0)
ESA_INST_FWD_D(float, 1)
ESA_INST_FWD_D(_Float16, 0)
ESA_INST_FWD_D(_Float16, 1)
ESA_INST_FWD_D(__bf16, 0)
ESA_INST_FWD_D(__bf16, 1)

}  // namespace esa
