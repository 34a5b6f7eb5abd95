// Backward of the ESA forward scan for gfx950: one pass over HBM that reads a, v, q, dy
// (and the forward's fp32 state checkpoint every 64 steps) and writes d_logit, d_value and
// d_query.
//
// The pages state no backward; it is the chain rule through the forward of page
// "entangled-state-attention 0.1.0", section "Core idea".  With n = E_t r_t and
// r_t = (mean_h E_t^2 + eps)^(-1/2):
//   readout   dq = dy n,  dn = dy q,  gE = r (dn - n mean_h(dn n))
//   reverse   dE_t = gE_t + lam_{t+1},  lam_t = s_t dE_t,  lam_T = dE_final, dE_init = lam_0
//   direct    d_logit = dE_t E_{t-1} s (1 - s),          d_value = dE_t
//   controlled d_logit = dE_t (E_{t-1} - v_t) s (1 - s), d_value = dE_t (1 - s)
// The reverse recurrence lam_t = s_t (gE_t + lam_{t+1}) is the same affine pair scan as
// the forward, run from the end of the sequence: workgroup IDs number tiles from the last one and
// look back toward later tiles.
//
// A tile first re-runs the forward inside itself from the checkpointed state at its start
// (level 1 and 2 of the forward scan, no look-back needed), keeping per element only what
// the reverse pass uses: s, gE, the gate-gradient factor w and, in controlled mode, 1 - s.
#include "esa_common.hpp"

namespace esa {

template <typename T, int MODE, int DH, int L, int NT>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
    using G = Geom<T, DH, L, NT>;
    constexpr int VEC = G::VEC, CB = G::CB, NCL = G::NCL, S = G::S, HL = G::HL;
    constexpr int TT = G::TT;
    constexpr int ES = sizeof(T);

    __shared__ float sP[S][CB];
    __shared__ float sE[S][CB];

    const uint32_t wg = blockIdx.x;
    const uint32_t rtile = wg / p.nCB;
    const uint32_t cb = wg - rtile * p.nCB;
    const uint32_t tile = p.nTiles - 1 - rtile;  // the backward walks tiles from the end
    const uint32_t tagAgg = make_tag(p.epoch, kTagAgg);
    const uint32_t tagInc = make_tag(p.epoch, kTagInc);

    const int tid = threadIdx.x;
    const int j = tid % NCL;
    const int slot = tid / NCL;
    const int64_t lane0 = (int64_t)cb * CB + j * VEC;
    const bool lane_ok = lane0 < p.nLanes;
    const int64_t b = lane_ok ? lane0 / p.C : 0;
    const int64_t c = lane_ok ? lane0 - b * p.C : 0;
    const int64_t t0 = (int64_t)tile * TT + (int64_t)slot * L;
    const int64_t base = (b * p.T + t0) * p.C + c;

    uint4 ra[L], rv[L], rq[L], rd[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        ra[i] = make_uint4(0, 0, 0, 0);
        rv[i] = make_uint4(0, 0, 0, 0);
        rq[i] = make_uint4(0, 0, 0, 0);
        rd[i] = make_uint4(0, 0, 0, 0);
        if (lane_ok && t0 + i < p.T) {
            ra[i] = ld16(p.a, base + i * p.C, ES);
            rv[i] = ld16(p.v, base + i * p.C, ES);
            rq[i] = ld16(p.q, base + i * p.C, ES);
            rd[i] = ld16(p.dy, base + i * p.C, ES);
        }
    }

    // ---- gates and the thread's forward fold ----
    // S_[i][e] = s; U_[i][e] = 1 - s (controlled) or s (1 - s) (direct); V_[i][e] = v
    float S_[L][VEC], U_[L][VEC], V_[L][VEC];
    float P[VEC], E[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        P[e] = 1.0f;
        E[e] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = lane_ok && t0 + i < p.T;
        float av[VEC];
        unpack<T>(ra[i], av);
        unpack<T>(rv[i], V_[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float s, u;
            gate(av[e], s, u);
            s = ok ? s : 1.0f;
            u = ok ? u : 0.0f;
            S_[i][e] = s;
            U_[i][e] = MODE == kDirect ? s * u : u;
            const float bt = MODE == kDirect ? (ok ? V_[i][e] : 0.0f) : u * V_[i][e];
            E[e] = s * E[e] + bt;
            P[e] = P[e] * s;
        }
    }

    // ---- forward prefix within the tile, from the checkpointed state at its start ----
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
            const int64_t gl = (int64_t)cb * CB + ch;
            float cin = 0.0f;
            if (gl < p.nLanes) {
                if (tile == 0) {
                    cin = p.e0 ? p.e0[gl] : 0.0f;
                } else {
                    const int64_t gb = gl / p.C, gc = gl - gb * p.C;
                    const int64_t ck = (int64_t)tile * (TT / kCkptChunk) - 1;
                    cin = p.ckpt[(gb * p.nck + ck) * p.C + gc];
                }
            }
            float te = cin;
#pragma unroll 8
            for (int s = 0; s < S; ++s) {
                const float ps = sP[s][ch], es = sE[s][ch];
                sE[s][ch] = te;  // state entering slot s
                te = ps * te + es;
            }
        }
    }
    __syncthreads();

    // ---- re-run the forward per step; readout backward; keep gE and the gate factor ----
    float Gr[L][VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) E[e] = sE[slot][j * VEC + e];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = lane_ok && t0 + i < p.T;
        float Eprev[VEC];
        float ss = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Eprev[e] = E[e];
            const float bt = MODE == kDirect ? (ok ? V_[i][e] : 0.0f) : U_[i][e] * V_[i][e];
            E[e] = S_[i][e] * E[e] + bt;
            ss += E[e] * E[e];
        }
        ss = head_sum<HL>(ss);
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DH) + kEps);
        float qv[VEC], dyv[VEC], n[VEC], dn[VEC], dqv[VEC];
        unpack<T>(rq[i], qv);
        unpack<T>(rd[i], dyv);
        float dd = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            n[e] = E[e] * r;
            dqv[e] = dyv[e] * n[e];
            dn[e] = dyv[e] * qv[e];
            dd += dn[e] * n[e];
        }
        dd = head_sum<HL>(dd);
        const float mu = dd * (1.0f / DH);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Gr[i][e] = ok ? r * (dn[e] - n[e] * mu) : 0.0f;
            // gate factor w, stored over V_: d_logit = dE * w
            const float su = MODE == kDirect ? U_[i][e] : S_[i][e] * U_[i][e];
            V_[i][e] = MODE == kDirect ? Eprev[e] * su : (Eprev[e] - V_[i][e]) * su;
        }
        if (ok) st16(p.dq, base + i * p.C, ES, pack<T>(dqv));
    }

    // ---- reverse fold of the thread's steps: lam_out = P * lam_in + E ----
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        float pr = 1.0f, er = 0.0f;
#pragma unroll
        for (int i = L - 1; i >= 0; --i) {
            er = S_[i][e] * (Gr[i][e] + er);
            pr = S_[i][e] * pr;
        }
        P[e] = pr;
        E[e] = er;
    }
    __syncthreads();  // every thread has read its forward prefix from sE
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
            for (int s = S - 1; s >= 0; --s) {
                const float ps = sP[s][ch], es = sE[s][ch];
                sP[s][ch] = tp;  // map from the tile's right edge to slot s's right edge
                sE[s][ch] = te;
                te = ps * te + es;
                tp = ps * tp;
            }
            const int64_t gl = (int64_t)cb * CB + ch;
            float carry = 0.0f;
            if (gl < p.nLanes) {
                uint64_t* X = p.flagX + (int64_t)tile * p.nLanes + gl;
                if (tile == p.nTiles - 1) {
                    carry = p.dET ? p.dET[gl] : 0.0f;
                } else {
                    publish(X, tagAgg, te);
                    publish(p.flagY + (int64_t)tile * p.nLanes + gl, tagAgg, tp);
                    carry = look_back(p.flagX, p.flagY, p.nLanes, gl, tile, +1, tagAgg, tagInc, p.hdr);
                }
                const float lam_out = te + tp * carry;
                publish(X, tagInc, lam_out);
                if (tile == 0 && p.de0) p.de0[gl] = lam_out;
            }
            // fold the carry into every slot's entry value
#pragma unroll 8
            for (int s = 0; s < S; ++s) sE[s][ch] = sE[s][ch] + sP[s][ch] * carry;
        }
    }
    __syncthreads();

    // ---- reverse recurrence over the thread's steps; gate and value gradients ----
    float lam[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) lam[e] = sE[slot][j * VEC + e];
#pragma unroll
    for (int i = L - 1; i >= 0; --i) {
        const bool ok = lane_ok && t0 + i < p.T;
        float dav[VEC], dvv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float dE = Gr[i][e] + lam[e];
            lam[e] = S_[i][e] * dE;
            dav[e] = dE * V_[i][e];
            dvv[e] = MODE == kDirect ? dE : dE * U_[i][e];
        }
        if (ok) {
            st16(p.da, base + i * p.C, ES, pack<T>(dav));
            st16(p.dv, base + i * p.C, ES, pack<T>(dvv));
        }
    }
}

template <typename T, int MODE, int DH>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
    using C = BwdCfg<T, DH>;
    hipLaunchKernelGGL((bwd_kernel<T, MODE, DH, C::L, C::NT>), dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
    return hipGetLastError();
}

#define ESA_INST_BWD(T, M, D) template hipError_t launch_bwd<T, M, D>(const BwdParams&, hipStream_t);
#define ESA_INST_BWD_D(T, M) \
    ESA_INST_BWD(T, M, 16) ESA_INST_BWD(T, M, 32) ESA_INST_BWD(T, M, 64) ESA_INST_BWD(T, M, 128)
ESA_INST_BWD_D(float, 0)
ESA_INST_BWD_D(float, 1)
ESA_INST_BWD_D(_Float16, 0)
ESA_INST_BWD_D(_Float16, 1)
ESA_INST_BWD_D(__bf16, 0)
ESA_INST_BWD_D(__bf16, 1)

}  // namespace esa
