// Forward scan of the ESA gated linear recurrence with fused gate and per-head RMSNorm
// readout, for gfx950.  One pass over HBM: a, v, q are read once and y is written once.
//
// Recurrence and gates: page "entangled-state-attention 0.1.0", section "Core idea" (direct
// and controlled ESA); readout y = q * Norm(E_t) from the same section, with Norm read as
// per-head RMSNorm (eps 1e-6, no gain); composition over the sequence and the compact final
// state: page "Entangled State Attention", section "[ ARCHITECTURE ]".
//
// Loads are issued without branches (rows past the end of the sequence and lanes past the
// end of the batch load a clamped, valid address and are masked afterwards), so all of a
// thread's loads are in flight at once; a branch between two loads would make the compiler
// drain the first before issuing the next.  Tiles that are entirely inside the problem (all
// but the ragged last tile row and channel block) take a path with no per-element masking,
// addressing every load as a workgroup-uniform base plus one 32-bit lane offset.
#include "esa_common.hpp"

namespace esa {

template <typename T, int MODE, int DH, int L, int NT, bool READOUT, bool PROD, bool FULL,
          int CHAIN>
__device__ __forceinline__ void fwd_tile(const FwdParams& p, uint32_t tile, uint32_t cb,
                                         Acc<T>* sP, Acc<T>* sE, Acc<T>* sWP, Acc<T>* sWE,
                                         Acc<T>* sCarry, float* sGate) {
    using G = Geom<T, DH, L, NT>;
    constexpr int VEC = G::VEC, CB = G::CB, NCL = G::NCL, HL = G::HL;
    constexpr int TT = G::TT;
    constexpr int ES = sizeof(T);
    // gate products are carried as complements (GP); the segment pass converts its gate
    // product output back to a product at the end.  F: the accumulation type (Acc).
    constexpr bool CQ = true;
    using F = Acc<T>;
    using Q = GP<CQ, F>;
    static_assert(kCkptChunk % L == 0, "checkpoint steps must end a thread's slot");
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
    uint4 ra[L], rv[L], rq[L];
    // full tiles: buffer resources at the tile's first element, one lane offset, row offsets
    const int64_t g0 = (int64_t)cb * CB;
    const int64_t bw = g0 / p.C;
    const int64_t row0 = ((bw * p.T + (int64_t)tile * TT) * p.C + (g0 - bw * p.C)) * ES;
    const uint32_t voff = (uint32_t)(((int64_t)slot * L * p.C + j * VEC) * ES);
    const int32_t rstride = (int32_t)(p.C * ES);
    if constexpr (FULL) {
        const auto rs_a = make_rsrc(static_cast<const char*>(p.a) + row0);
        const auto rs_v = make_rsrc(static_cast<const char*>(p.v) + row0);
#pragma unroll
        for (int i = 0; i < L; ++i) {
            ra[i] = ldbuf<T>(rs_a, voff, i * rstride);
            rv[i] = ldbuf<T>(rs_v, voff, i * rstride);
            if constexpr (READOUT) rq[i] = ldbuf<T>(make_rsrc(static_cast<const char*>(p.q) + row0), voff, i * rstride);
            else rq[i] = make_uint4(0, 0, 0, 0);
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
            if constexpr (READOUT) rq[i] = ld16<T>(p.q, off, ES);
            else rq[i] = make_uint4(0, 0, 0, 0);
        }
    }

    // one-byte storage: the gate table (kGateTable), filled while the loads are in flight
    constexpr bool TAB = kGateTable<T>;
    if constexpr (TAB) {
        fill_gate_table<T, NT>(sGate);
        __syncthreads();
    }

    // ---- level 1: gates and the thread's own fold (identity step where masked) ----
    // Each step is x' = s x + b (update()).  With fp32 accumulation SB[i] holds s = 1 - u and
    // WB[i] the write term b, so the re-run below is one fma per step; with fp64 accumulation
    // they hold u and v, and s and b are formed in fp64 at each use (an fp32 s would round).
    // A masked step holds s = 1, b = 0 (u = 0, v = 0).  One-byte storage does not keep them
    // (REDO below).
    constexpr bool WIDE = std::is_same<F, double>::value;
    float SB[L][VEC], WB[L][VEC];
    F P[VEC], E[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        P[e] = Q::one;
        E[e] = F(0);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const bool ok = FULL || (lane_ok && t0 + i < p.T);
        float av[VEC], vv[VEC];
        if constexpr (TAB)
            gate_u_lookup(ra[i], sGate, av);
        else
            unpack<T>(ra[i], av);
        unpack<T>(rv[i], vv);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float u = ok ? (TAB ? av[e] : gate_u(av[e])) : 0.0f;
            const float v = ok ? vv[e] : 0.0f;
            const F s = F(1) - F(u), b = step_b<MODE, F>(F(u), F(v));
            SB[i][e] = WIDE ? u : float(s);
            WB[i][e] = WIDE ? v : float(b);
            E[e] = update<F>(E[e], s, b);
            P[e] = i == 0 ? F(u) : fma_(P[e], s, F(u));  // Q::mul(P, u) with s = 1 - u
        }
    }

    // ---- level 2: slot pairs through LDS (within each wave, then across the waves) ----
    const int w = tid / kWave;
    F xp[G::CPL][G::SPW], xe[G::CPL][G::SPW];
    slots_phase_a<G, false, CQ, F>(P, E, sP, sE, sWP, sWE, xp, xe);
    __syncthreads();
    slots_phase_b<G, false, CQ, F>(sP, sE, sWP, sWE, xp, xe);

    // ---- level 3: decoupled look-back across tiles, wave k for channels 64k.. (lane = channel) ----
    if (w < G::CPL) {
        const int ch = (tid % kWave) + w * kWave;
        F tp, te;
        tile_total<G, false, CQ, F>(sWP, sWE, ch, tp, te);
        const int64_t gl = (int64_t)cb * CB + ch;
        F carry = F(0);
        constexpr bool STATS = CHAIN == kChainStats;
        WalkCount wc{~0u, 0u};  // statistics instance: set when the lane walked back
        bool active = false;
        if (FULL || gl < p.nLanes) {
            uint64_t* X = p.flagX + (int64_t)tile * p.nLanes + gl;
            uint64_t* Y = p.flagY + (int64_t)tile * p.nLanes + gl;
            float pin = GP<CQ>::one;  // PROD: product of the gates of every earlier tile
            constexpr bool TEST = CHAIN == kChainTest;
            const uint32_t det = CHAIN == kChainDet || TEST ? p.det : 0u;
            const bool inc = det_publishes_inc(tile, det);
            if (tile == 0) {
                carry = p.e0 ? p.e0[gl] : 0.0f;
            } else {
                active = true;
                carry = chain_carry<PROD, TEST ? kTestSpinLimit : kSpinLimit, CQ, F>(
                    p.flagX, p.flagY, p.nLanes, gl, tile, -1, tagAgg, tagInc, p.hdr, float(tp),
                    float(te), &pin, det, inc, STATS ? &wc : nullptr);
            }
            // the test instance withholds tile 0
            const bool pub = (!TEST || tile != 0) && inc;
            if constexpr (PROD) {
                const F prod = Q::mul(tp, F(pin));
                if (pub) publish(Y, tagInc, float(prod));
                if (tile == p.nTiles - 1) p.prod[gl] = float(CQ ? F(1) - prod : prod);
            }
            if (pub) publish(X, tagInc, float(Q::comp(tp, F(carry), te)));
        }
        if constexpr (STATS) count_walks(p.hdr, active, wc.folded != ~0u, wc);
        sCarry[ch] = carry;
    }
    __syncthreads();

    if constexpr (!READOUT) {
        // State-only pass (checkpoint, final state, gate product): no step needs its own state,
        // so the thread applies its folded pair to the state entering its slot.  Checkpoint
        // steps (t % 64 == 63) and the sequence's last step always end a slot, because 64 is
        // a multiple of L and masked steps are the identity.  This skips the per-step re-run
        // and the per-step gate arrays (measured 13 % faster at 64K context).
        F XP[VEC], XE[VEC];
        read_exclusive<G>(sP, sE, XP, XE);
        const int64_t tend = (t0 + L < p.T ? t0 + L : p.T) - 1;
        if ((FULL || lane_ok) && t0 < p.T) {
            float Ef[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                Ef[e] = float(Q::comp(P[e], Q::comp(XP[e], F(sCarry[j * VEC + e]), XE[e]), E[e]));
            if (p.ckpt && (((tend + 1) % kCkptChunk) == 0 || tend == p.T - 1)) {
                float* dst = p.ckpt + (b * p.nck + tend / kCkptChunk) * p.C + c;
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<float4*>(dst + e) = make_float4(Ef[e], Ef[e + 1], Ef[e + 2], Ef[e + 3]);
            }
            if (p.eT && tend == p.T - 1) {
                float* dst = p.eT + lane0;
#pragma unroll
                for (int e = 0; e < VEC; e += 4)
                    *reinterpret_cast<float4*>(dst + e) = make_float4(Ef[e], Ef[e + 1], Ef[e + 2], Ef[e + 3]);
            }
        }
        return;
    }

    // ---- carry in, re-run the recurrence, readout ----
    {
        F XP[VEC], XE[VEC];
        read_exclusive<G>(sP, sE, XP, XE);
#pragma unroll
        for (int e = 0; e < VEC; ++e) E[e] = Q::comp(XP[e], F(sCarry[j * VEC + e]), XE[e]);
    }
    const int64_t ckbase = b * p.nck;
    // One-byte storage re-derives each step's gate from the raw words through the gate table
    // instead of keeping SB and WB: 77 rather than 112 VGPRs, three workgroups per CU rather
    // than two.  This forward is bound by its vector ALU, so the controlled step takes the
    // two-instruction form E + u (v - E), equal to s E + u v up to rounding: one rounding of
    // v - E, scaled by u, and one of the result (E, a convex combination of the initial state
    // and the values, keeps v - E on their scale).  The empty asm hides the words' values
    // from the compiler, which would otherwise keep the fold's results alive instead of
    // recomputing them; one statement covers the four steps' words (words x, y: the upper two
    // of a one-byte load are zero), as per-step statements compiled to 103 VGPRs.
    constexpr bool REDO = TAB && !WIDE;
    if constexpr (REDO) {
        static_assert(L == 4, "the re-derived steps hide four steps' words in one statement");
        asm volatile("" : "+v"(ra[0].x), "+v"(ra[0].y), "+v"(rv[0].x), "+v"(rv[0].y),
                          "+v"(ra[1].x), "+v"(ra[1].y), "+v"(rv[1].x), "+v"(rv[1].y),
                          "+v"(ra[2].x), "+v"(ra[2].y), "+v"(rv[2].x), "+v"(rv[2].y),
                          "+v"(ra[3].x), "+v"(ra[3].y), "+v"(rv[3].x), "+v"(rv[3].y));
    }
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int64_t t = t0 + i;
        const bool ok = FULL || (lane_ok && t < p.T);
        float ss = 0.0f, Ef[VEC];
        float ru[VEC], rw[VEC];
        if constexpr (REDO) {
            gate_u_lookup(ra[i], sGate, ru);
            unpack<T>(rv[i], rw);
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (REDO) {
                const float u = ok ? ru[e] : 0.0f, v = ok ? rw[e] : 0.0f;
                if constexpr (MODE == kControlled)
                    E[e] = fma_(F(u), F(v) - E[e], E[e]);
                else
                    E[e] = update<F>(E[e], F(1) - F(u), F(v));
            } else if constexpr (WIDE)
                E[e] = update<F>(E[e], F(1) - F(SB[i][e]), step_b<MODE, F>(F(SB[i][e]), F(WB[i][e])));
            else
                E[e] = update<F>(E[e], F(SB[i][e]), F(WB[i][e]));
            Ef[e] = float(E[e]);
            ss += Ef[e] * Ef[e];
        }
        if constexpr (READOUT) {
            ss = head_sum<HL>(ss);
            const float r = __builtin_amdgcn_rsqf(ss * (1.0f / DH) + kEps);
            float qv[VEC], yv[VEC];
            unpack<T>(rq[i], qv);
#pragma unroll
            for (int e = 0; e < VEC; ++e) yv[e] = qv[e] * (Ef[e] * r);
            if constexpr (FULL)
                stbuf<T>(static_cast<char*>(p.y) + row0 + i * rstride, voff, pack<T>(yv));
            else if (ok)
                st16<T>(p.y, base + i * p.C, ES, pack<T>(yv));
        }
        if (ok && p.ckpt && (((t + 1) % kCkptChunk) == 0 || t == p.T - 1)) {
            float* dst = p.ckpt + (ckbase + t / kCkptChunk) * p.C + c;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(Ef[e], Ef[e + 1], Ef[e + 2], Ef[e + 3]);
        }
        if (ok && p.eT && t == p.T - 1) {
            float* dst = p.eT + lane0;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4*>(dst + e) = make_float4(Ef[e], Ef[e + 1], Ef[e + 2], Ef[e + 3]);
        }
    }
}

template <typename T, int MODE, int DH, int L, int NT, bool READOUT, bool PROD, int CHAIN>
__global__ __launch_bounds__(NT) void fwd_kernel(FwdParams p) {
    static_assert(!(READOUT && PROD), "the gate product comes from the state-only pass");
    using G = Geom<T, DH, L, NT>;
    constexpr int CB = G::CB, TT = G::TT, NW = G::NW, S = G::S;
    using F = Acc<T>;
    __shared__ __attribute__((aligned(16))) F sP[S * CB];  // per-slot pairs
    __shared__ __attribute__((aligned(16))) F sE[S * CB];
    __shared__ F sWP[NW * CB];  // per-wave aggregate pairs
    __shared__ F sWE[NW * CB];
    __shared__ F sCarry[CB];
    float* sGate = nullptr;
    if constexpr (kGateTable<T>) {
        __shared__ float gateTable[256];
        sGate = gateTable;
    }

    uint32_t tile, cb;
    tile_of(blockIdx.x, p.nCB, tile, cb);
    // full: every step and lane of the tile exists and its channel block lies in one batch row
    // (and the tile's byte span fits the 32-bit lane offsets)
    const bool full = (int64_t)(tile + 1) * TT <= p.T && (int64_t)(cb + 1) * CB <= p.nLanes &&
                      p.C % CB == 0 && (int64_t)TT * p.C * (int64_t)sizeof(T) < (int64_t(1) << 31);
    if (full)
        fwd_tile<T, MODE, DH, L, NT, READOUT, PROD, true, CHAIN>(p, tile, cb, sP, sE, sWP, sWE,
                                                                 sCarry, sGate);
    else
        fwd_tile<T, MODE, DH, L, NT, READOUT, PROD, false, CHAIN>(p, tile, cb, sP, sE, sWP, sWE,
                                                                  sCarry, sGate);
}

template <typename T, int MODE, int DH, int CHAIN, int V = 0>
hipError_t launch_fwd_as(const FwdParams& p, hipStream_t s) {
    using C = FwdCfg<T, DH, V>;
    const dim3 grid(p.nCB * p.nTiles), block(C::NT);
    if (p.y)
        hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT, true, false, CHAIN>), grid, block,
                           0, s, p);
    else if (p.prod)
        hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT, false, true, CHAIN>), grid, block,
                           0, s, p);
    else
        hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT, false, false, CHAIN>), grid, block,
                           0, s, p);
    return hipGetLastError();
}

template <typename T, int MODE, int DH>
hipError_t launch_fwd(const FwdParams& p, hipStream_t s) {
    if (p.y && p.withhold) {
        // the forced-timeout test instance exists for fp16 storage and Dh = 64 only (the host
        // rejects the flag for other problems)
        if constexpr (std::is_same<T, _Float16>::value && DH == 64) {
            using C = FwdCfg<T, DH>;
            hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT, true, false, kChainTest>),
                               dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
            return hipGetLastError();
        } else {
            return hipErrorNotSupported;
        }
    }
    if (p.y && p.stats) {
        // the look-back statistics instance: fp16 and fp8 E4M3 storage with Dh = 64 (the host
        // rejects the flag for other problems)
        if constexpr ((std::is_same<T, _Float16>::value || std::is_same<T, f8e4m3>::value) &&
                      DH == 64) {
            using C = FwdCfg<T, DH>;
            hipLaunchKernelGGL((fwd_kernel<T, MODE, DH, C::L, C::NT, true, false, kChainStats>),
                               dim3(p.nCB * p.nTiles), dim3(C::NT), 0, s, p);
            return hipGetLastError();
        } else {
            return hipErrorNotSupported;
        }
    }
    if constexpr (kHasFwdVariant<T, DH>) {
        if (p.variant == 1)
            return p.det ? launch_fwd_as<T, MODE, DH, kChainDet, 1>(p, s)
                         : launch_fwd_as<T, MODE, DH, kChainDefault, 1>(p, s);
    }
    if (p.variant != 0) return hipErrorNotSupported;
    return p.det ? launch_fwd_as<T, MODE, DH, kChainDet>(p, s)
                 : launch_fwd_as<T, MODE, DH, kChainDefault>(p, s);
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
ESA_INST_FWD_D(f8e4m3, 0)
ESA_INST_FWD_D(f8e4m3, 1)
ESA_INST_FWD_D(f8e5m2, 0)
ESA_INST_FWD_D(f8e5m2, 1)

}  // namespace esa
