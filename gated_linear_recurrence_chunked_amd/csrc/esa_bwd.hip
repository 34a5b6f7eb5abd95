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
// As in the forward, every load is issued branch-free at a clamped, valid address, and
// tiles entirely inside the problem skip the per-element masking and address their loads
// and stores through buffer resources with one 32-bit lane offset.
#include "esa_common.hpp"

namespace esa {

template <typename T, int MODE, int DH, int L, int NT, bool GRADS, bool FULL, int CHAIN>
__device__ __forceinline__ void bwd_tile(const BwdParams& p, uint32_t tile, uint32_t cb,
                                         Acc<T>* sP, Acc<T>* sE, Acc<T>* sWP, Acc<T>* sWE,
                                         Acc<T>* sCarry, float* sGate) {
    using G = Geom<T, DH, L, NT>;
    constexpr int VEC = G::VEC, CB = G::CB, NCL = G::NCL, HL = G::HL;
    constexpr int TT = G::TT;
    constexpr int ES = sizeof(T);
    constexpr bool CQ = true;  // gate products are carried as complements (GP)
    using F = Acc<T>;          // the accumulation type (Acc)
    using Q = GP<CQ, F>;
    const uint32_t epoch = launch_epoch(p.epoch, p.epochWord);
    const uint32_t tagAgg = make_tag(epoch, kTagAgg);
    const uint32_t tagInc = make_tag(epoch, kTagInc);

    const int tid = threadIdx.x;
    const int j = tid % NCL;
    const int slot = tid / NCL;
    const int64_t lane0 = (int64_t)cb * CB + j * VEC;
    const bool lane_ok = FULL || lane0 < p.nLanes;
    const int64_t b = lane_ok ? lane0 / p.C : 0;
    const int64_t c = lane_ok ? lane0 - b * p.C : 0;
    const int64_t t0 = (int64_t)tile * TT + (int64_t)slot * L;
    const int64_t base = (b * p.T + t0) * p.C + c;

    // ---- issue every load of the thread's L steps, branch-free ----
    uint4 ra[L], rv[L], rq[L], rd[L];
    // full tiles: buffer resources at the tile's first element, one lane offset, row offsets
    const int64_t g0 = (int64_t)cb * CB;
    const int64_t bw = g0 / p.C;
    const int64_t row0 = ((bw * p.T + (int64_t)tile * TT) * p.C + (g0 - bw * p.C)) * ES;
    const uint32_t voff = (uint32_t)(((int64_t)slot * L * p.C + j * VEC) * ES);
    const int32_t rstride = (int32_t)(p.C * ES);
    if constexpr (FULL) {
        const auto rs_a = make_rsrc(static_cast<const char*>(p.a) + row0);
        const auto rs_v = make_rsrc(static_cast<const char*>(p.v) + row0);
        const auto rs_q = make_rsrc(static_cast<const char*>(p.q) + row0);
        const auto rs_d = make_rsrc(static_cast<const char*>(p.dy) + row0);
#pragma unroll
        for (int i = 0; i < L; ++i) {
            ra[i] = ldbuf<T>(rs_a, voff, i * rstride);
            rv[i] = ldbuf<T>(rs_v, voff, i * rstride);
            rq[i] = ldbuf<T>(rs_q, voff, i * rstride);
            rd[i] = ldbuf<T>(rs_d, voff, i * rstride);
        }
    } else {
        // ragged tile: rows past the end and lanes past the batch load a clamped, valid
        // address and are masked below
        const int64_t lc = lane_ok ? lane0 : 0;
        const int64_t bc = lc / p.C, cc = lc - bc * p.C;
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int64_t t = t0 + i < p.T ? t0 + i : p.T - 1;
            const int64_t off = (bc * p.T + t) * p.C + cc;
            ra[i] = ld16<T>(p.a, off, ES);
            rv[i] = ld16<T>(p.v, off, ES);
            rq[i] = ld16<T>(p.q, off, ES);
            rd[i] = ld16<T>(p.dy, off, ES);
        }
    }
    // state entering the tile: the initial state, or the forward's checkpoint at the end of
    // the previous 64-step chunk (masked lanes read a valid lane's value, then stay masked)
    float cin[VEC];
    {
        const int64_t lc = lane_ok ? lane0 : 0;
        const int64_t bc = lc / p.C, cc = lc - bc * p.C;
        const float* src =
            tile == 0 ? (p.e0 ? p.e0 + lc : nullptr)
                      : p.ckpt + (bc * p.nck + (int64_t)tile * (TT / kCkptChunk) - 1) * p.C + cc;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
            float4 x = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (src) x = *reinterpret_cast<const float4*>(src + e);
            cin[e] = x.x;
            cin[e + 1] = x.y;
            cin[e + 2] = x.z;
            cin[e + 3] = x.w;
        }
    }

    // one-byte storage, full tiles: the gate table (kGateTable), filled while the loads are in
    // flight (ragged tiles evaluate the gate in place: there the table raised the kernel's
    // register peak from 232 to 265 VGPRs, one wave per SIMD)
    constexpr bool TAB = kGateTable<T> && FULL;
    if constexpr (TAB) {
        fill_gate_table<T, NT>(sGate);
        __syncthreads();
    }

    // ---- gates and the thread's forward fold ----
    // S_[i][e] = 1 - s (the complement, GP); V_[i][e] = v (masked steps: 0 and 0, the
    // identity); with fp32 storage also U_[i][e] = s (1 - s) (gate_u_slope)
    constexpr bool SLOPE = sizeof(T) == 4;
    float S_[L][VEC], V_[L][VEC], U_[SLOPE ? L : 1][VEC];
    F P[VEC], E[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        P[e] = Q::one;
        E[e] = F(0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = FULL || (lane_ok && t0 + i < p.T);
        float av[VEC];
        if constexpr (TAB)
            gate_u_lookup(ra[i], sGate, av);
        else
            unpack<T>(ra[i], av);
        unpack<T>(rv[i], V_[i]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float u;
            if constexpr (SLOPE) {
                float su;
                u = gate_u_slope(av[e], su);
                U_[i][e] = ok ? su : 0.0f;
            } else {
                u = TAB ? av[e] : gate_u(av[e]);
            }
            S_[i][e] = ok ? u : 0.0f;
            V_[i][e] = ok ? V_[i][e] : 0.0f;
            const F s = F(1) - F(S_[i][e]);
            E[e] = update<F>(E[e], s, step_b<MODE, F>(F(S_[i][e]), F(V_[i][e])));
            P[e] = i == 0 ? F(S_[i][e]) : fma_(P[e], s, F(S_[i][e]));  // Q::mul(P, u)
        }
    }

    // ---- state entering this thread's steps: the checkpoint at the tile start, carried
    //      through the earlier slots of the tile (two-phase slot scan, no look-back needed) ----
    const int w = tid / kWave;
    F xp[G::CPL][G::SPW], xe[G::CPL][G::SPW];
    F XP[VEC], XE[VEC];
    slots_phase_a<G, false, CQ, F>(P, E, sP, sE, sWP, sWE, xp, xe);
    __syncthreads();
    slots_phase_b<G, false, CQ, F>(sP, sE, sWP, sWE, xp, xe);
    __syncthreads();
    read_exclusive<G>(sP, sE, XP, XE);
#pragma unroll
    for (int e = 0; e < VEC; ++e) E[e] = Q::comp(XP[e], F(cin[e]), XE[e]);

    // ---- re-run the forward per step; readout backward; keep gE and the gate factor ----
    float Gr[L][VEC];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = FULL || (lane_ok && t0 + i < p.T);
        F Eprev[VEC];
        float ss = 0.0f, Ef[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            Eprev[e] = E[e];
            E[e] = update<F>(E[e], F(1) - F(S_[i][e]), step_b<MODE, F>(F(S_[i][e]), F(V_[i][e])));
            Ef[e] = float(E[e]);
            ss += Ef[e] * Ef[e];
        }
        ss = head_sum<HL>(ss);
        const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DH) + kEps);
        float qv[VEC], dyv[VEC], n[VEC], dn[VEC], dqv[VEC];
        unpack<T>(rq[i], qv);
        unpack<T>(rd[i], dyv);
        float dd = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            n[e] = Ef[e] * r;
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
            float su;  // s (1 - s)
            if constexpr (SLOPE) su = U_[i][e];
            else su = gate_slope(S_[i][e]);
            V_[i][e] = float(MODE == kDirect ? Eprev[e] * F(su) : (Eprev[e] - F(V_[i][e])) * F(su));
        }
        if constexpr (GRADS) {
            if constexpr (FULL)
                stbuf<T>(static_cast<char*>(p.dq) + row0 + i * rstride, voff, pack<T>(dqv));
            else if (ok)
                st16<T>(p.dq, base + i * p.C, ES, pack<T>(dqv));
        }
    }

    // ---- reverse fold of the thread's steps: lam_out = P * lam_in + E ----
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        F pr = Q::one, er = F(0);
#pragma unroll
        for (int i = L - 1; i >= 0; --i) {
            er = Q::apply(F(S_[i][e]), F(Gr[i][e]) + er);
            pr = i == L - 1 ? F(S_[i][e]) : Q::mul(pr, F(S_[i][e]));
        }
        P[e] = pr;
        E[e] = er;
    }
    // the slot arrays are reused: this thread's slot positions were last read by this thread,
    // and the wave aggregates by every wave before the barrier above
    slots_phase_a<G, true, CQ, F>(P, E, sP, sE, sWP, sWE, xp, xe);
    __syncthreads();
    slots_phase_b<G, true, CQ, F>(sP, sE, sWP, sWE, xp, xe);

    // ---- reverse look-back across tiles, wave k for channels 64k.. (lane = channel) ----
    if (w < G::CPL) {
        const int ch = (tid % kWave) + w * kWave;
        F tp, te;
        tile_total<G, true, CQ, F>(sWP, sWE, ch, tp, te);
        const int64_t gl = (int64_t)cb * CB + ch;
        F carry = F(0);
        constexpr bool STATS = CHAIN == kChainStats;
        WalkCount wc{~0u, 0u};  // statistics instance: set when the lane walked back
        bool active = false;
        if (FULL || gl < p.nLanes) {
            uint64_t* X = p.flagX + (int64_t)tile * p.nLanes + gl;
            constexpr bool TEST = CHAIN == kChainTest;
            const uint32_t det = CHAIN == kChainDet || TEST ? p.det : 0u;
            const bool inc = det_publishes_inc(p.nTiles - 1 - tile, det);
            if (tile == p.nTiles - 1) {
                carry = p.dET ? p.dET[gl] : 0.0f;
            } else {
                float pin;  // unused: the backward carries no gate product
                active = true;
                carry = chain_carry<false, TEST ? kTestSpinLimit : kSpinLimit, CQ, F>(
                    p.flagX, p.flagY, p.nLanes, gl, tile, +1, tagAgg, tagInc, p.hdr, float(tp),
                    float(te), &pin, det, inc, STATS ? &wc : nullptr);
            }
            const float lam_out = float(Q::comp(tp, F(carry), te));
            // the test instance withholds the last tile
            if ((!TEST || tile != p.nTiles - 1) && inc) publish(X, tagInc, lam_out);
            if (tile == 0 && p.de0) p.de0[gl] = lam_out;
        }
        if constexpr (STATS) count_walks(p.hdr, active, wc.folded != ~0u, wc);
        sCarry[ch] = carry;
    }
    __syncthreads();
    read_exclusive<G>(sP, sE, XP, XE);

    // ---- reverse recurrence over the thread's steps; gate and value gradients ----
    F lam[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) lam[e] = Q::comp(XP[e], F(sCarry[j * VEC + e]), XE[e]);
#pragma unroll
    for (int i = L - 1; i >= 0; --i) {
        const bool ok = FULL || (lane_ok && t0 + i < p.T);
        float dav[VEC], dvv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const F dE = F(Gr[i][e]) + lam[e];
            lam[e] = Q::apply(F(S_[i][e]), dE);
            dav[e] = float(dE * F(V_[i][e]));
            dvv[e] = float(MODE == kDirect ? dE : dE * F(S_[i][e]));
        }
        if constexpr (GRADS) {
            if constexpr (FULL) {
                stbuf<T>(static_cast<char*>(p.da) + row0 + i * rstride, voff, pack<T>(dav));
                stbuf<T>(static_cast<char*>(p.dv) + row0 + i * rstride, voff, pack<T>(dvv));
            } else if (ok) {
                st16<T>(p.da, base + i * p.C, ES, pack<T>(dav));
                st16<T>(p.dv, base + i * p.C, ES, pack<T>(dvv));
            }
        }
    }
}

template <typename T, int MODE, int DH, int L, int NT, bool GRADS, int CHAIN>
__global__ __launch_bounds__(NT) void bwd_kernel(BwdParams p) {
    using G = Geom<T, DH, L, NT>;
    constexpr int CB = G::CB, TT = G::TT, NW = G::NW;
    using F = Acc<T>;
    __shared__ __attribute__((aligned(16))) F sP[G::S * CB];  // per-slot pairs / maps
    __shared__ __attribute__((aligned(16))) F sE[G::S * CB];
    __shared__ F sWP[NW * CB];  // per-wave aggregates
    __shared__ F sWE[NW * CB];
    __shared__ F sCarry[CB];
    float* sGate = nullptr;
    if constexpr (kGateTable<T>) {
        __shared__ float gateTable[256];
        sGate = gateTable;
    }

    uint32_t rtile, cb;
    tile_of(blockIdx.x, p.nCB, rtile, cb);
    const uint32_t tile = p.nTiles - 1 - rtile;  // the backward walks tiles from the end
    // full: every step and lane of the tile exists, its channel block lies in one batch row,
    // and the tile's byte span fits the 32-bit lane offsets
    const bool full = (int64_t)(tile + 1) * TT <= p.T && (int64_t)(cb + 1) * CB <= p.nLanes &&
                      p.C % CB == 0 && (int64_t)TT * p.C * (int64_t)sizeof(T) < (int64_t(1) << 31);
    if (full)
        bwd_tile<T, MODE, DH, L, NT, GRADS, true, CHAIN>(p, tile, cb, sP, sE, sWP, sWE, sCarry,
                                                         sGate);
    else
        bwd_tile<T, MODE, DH, L, NT, GRADS, false, CHAIN>(p, tile, cb, sP, sE, sWP, sWE, sCarry,
                                                          sGate);
}

template <typename T, int MODE, int DH, int CHAIN>
hipError_t launch_bwd_as(const BwdParams& p, hipStream_t s) {
    using C = BwdCfg<T, DH>;
    const dim3 grid(p.nCB * p.nTiles), block(C::NT);
    if (p.da)
        hipLaunchKernelGGL((bwd_kernel<T, MODE, DH, C::L, C::NT, true, CHAIN>), grid, block, 0, s,
                           p);
    else
        hipLaunchKernelGGL((bwd_kernel<T, MODE, DH, C::L, C::NT, false, CHAIN>), grid, block, 0, s,
                           p);
    return hipGetLastError();
}

template <typename T, int MODE, int DH>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s) {
    if (p.da && p.withhold) {
        // the forced-timeout test instance: fp16 storage and Dh = 64 only (as the forward)
        if constexpr (std::is_same<T, _Float16>::value && DH == 64) {
            using C = BwdCfg<T, DH>;
            hipLaunchKernelGGL((bwd_kernel<T, MODE, DH, C::L, C::NT, true, kChainTest>),
                               dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
            return hipGetLastError();
        } else {
            return hipErrorNotSupported;
        }
    }
    if (p.da && p.stats) {
        // the look-back statistics instance: fp16 and fp8 E4M3 storage with Dh = 64
        if constexpr ((std::is_same<T, _Float16>::value || std::is_same<T, f8e4m3>::value) &&
                      DH == 64) {
            using C = BwdCfg<T, DH>;
            hipLaunchKernelGGL((bwd_kernel<T, MODE, DH, C::L, C::NT, true, kChainStats>),
                               dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
            return hipGetLastError();
        } else {
            return hipErrorNotSupported;
        }
    }
    return p.det ? launch_bwd_as<T, MODE, DH, kChainDet>(p, s)
                 : launch_bwd_as<T, MODE, DH, kChainDefault>(p, s);
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
ESA_INST_BWD_D(f8e4m3, 0)
ESA_INST_BWD_D(f8e4m3, 1)
ESA_INST_BWD_D(f8e5m2, 0)
ESA_INST_BWD_D(f8e5m2, 1)

}  // namespace esa
