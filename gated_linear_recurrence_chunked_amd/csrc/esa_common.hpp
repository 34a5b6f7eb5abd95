// Shared definitions of the gfx950 kernels and the host dispatcher of libesa.so.
//
// The kernels scan E_t = A_t * E_{t-1} + B_t over T for every (b, h, d) lane of a
// [B, T, H, Dh] problem (page "Entangled State Attention v2.1", introduction; gates and
// readout from page "entangled-state-attention 0.1.0", "Core idea").  The scan is an exact
// re-association of the sequential loop through the pair combine
// (P1, E1) o (P2, E2) = (P1 P2, E2 + P2 E1) (page "Entangled State Attention",
// "[ ARCHITECTURE ]", associative composition):
//
//   lanes    a thread owns VEC channels (16 bytes of storage, 8 for one-byte storage) of
//            one (b, t); CB channels
//            (whole heads, at least 64 channels and 128 bytes) form a channel block,
//            NCL = CB / VEC threads wide.
//   tile     a workgroup owns one channel block over TT = S * L time steps: S time slots
//            of L consecutive steps, one slot per row of NCL threads.
//   level 1  each thread folds its L steps in registers into one pair per channel.
//   level 2  slot pairs go through LDS: lane = channel of each wave scans that wave's slots,
//            then the waves' aggregates are composed (slots_phase_a / slots_phase_b).
//   level 3  tiles of one channel block are chained by a decoupled look-back: a tile
//            whose neighbour already shows an inclusive value takes it; otherwise it
//            publishes its aggregate pair and walks back over earlier tiles' published
//            pairs until it meets an inclusive value.  Either way it then publishes its
//            own inclusive value.  For bitwise reproducible results only fixed positions
//            of the chain publish inclusive values (see chain_carry), so every carry folds
//            the same pairs on every run.
//   fp32     storage carries every gate product as its complement 1 - P (see GP).
//
// Tile order.  Workgroup IDs are tile-major within each XCD (see tile_of; the backward numbers
// tiles from the end), so a tile only ever waits on tiles with smaller IDs.  The hardware
// starts the workgroups of one dispatch in increasing ID order on each XCD, so the lowest
// unfinished workgroup is always resident and everything it waits on has finished: the chain
// always makes progress, with no atomic counter per workgroup (a single-address device atomic
// serialises at tens of ns each, which at 2^18 tiles would cost milliseconds).  Every wait is
// also bounded (see look_back), so even a broken chain ends.
//
// Look-back words are 64-bit (tag, fp32 value) pairs written and read with single-copy
// atomic 64-bit accesses at agent scope, so no fence is needed between a value and its
// flag.  The tag carries a per-launch epoch, so stale words from earlier launches never
// match and the flag array needs no clearing between calls.  An eagerly issued launch takes
// its epoch from a host counter; a launch recorded into a graph cannot (every replay would
// reuse the recorded value and find the previous replay's words), so it reads the epoch
// from the workspace header, where a one-thread kernel recorded just before it advances it
// on every replay.  The two kinds of epoch never coincide (bit 29 clear for host epochs,
// set for device epochs).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace esa {

constexpr int kWave = 64;
constexpr int kCkptChunk = 64;  // state checkpoint every 64 steps
constexpr float kEps = 1e-6f;   // RMSNorm epsilon (fixed reading of the pages' Norm)
constexpr int kDirect = 0;
constexpr int kControlled = 1;

template <typename T>
struct Storage;
template <>
struct Storage<float> {
    static constexpr int VEC = 4;
};
template <>
struct Storage<_Float16> {
    static constexpr int VEC = 8;
};
template <>
struct Storage<__bf16> {
    static constexpr int VEC = 8;
};
// One-byte floating-point storage in the two OCP 8-bit formats: E4M3 (4 exponent bits, bias
// 7, no infinities, max 448) and E5M2 (5 exponent bits, bias 15, IEEE-style infinities, max
// 57344).  The kernels decode them exactly to fp32 and round results back to nearest even
// with the gfx950 conversion instructions.
struct f8e4m3 {
    uint8_t bits;
};
struct f8e5m2 {
    uint8_t bits;
};
template <>
struct Storage<f8e4m3> {
    static constexpr int VEC = 8;
};
template <>
struct Storage<f8e5m2> {
    static constexpr int VEC = 8;
};
// Bytes of storage per thread and step: 16 (fp32, fp16, bf16) or 8 (fp8).
template <typename T>
constexpr int kVB = Storage<T>::VEC * (int)sizeof(T);

// Tile geometry of a scan kernel instance.  A channel block spans at least 64 channels and at
// least 128 bytes of each time row: with one-byte storage a 64-channel row piece is 64 bytes,
// and rows read in 64-byte pieces stream at about two thirds of the rate of 128-byte pieces.
template <typename T, int DH, int L, int NT>
struct Geom {
    static constexpr int VEC = Storage<T>::VEC;
    static constexpr int CBMIN = 128 / (int)sizeof(T) > 64 ? 128 / (int)sizeof(T) : 64;
    static constexpr int CB = DH > CBMIN ? DH : CBMIN;  // channels per block (whole heads)
    static constexpr int NCL = CB / VEC;          // threads across one time row
    static constexpr int S = NT / NCL;            // time slots per tile
    static constexpr int TT = S * L;              // time steps per tile
    static constexpr int HL = DH / VEC;           // threads per head
    static constexpr int CPL = CB / kWave;        // channels per lane in the slot scans, and
                                                  // look-back waves (one per 64 channels)
    static constexpr int NW = NT / kWave;         // waves per workgroup
    static constexpr int SPW = kWave / NCL;       // time slots per wave
    static_assert(CB % VEC == 0 && NT % NCL == 0 && S >= 1, "bad tile geometry");
    static_assert(kWave % NCL == 0 && CB % kWave == 0, "a wave holds whole rows of a block");
    static_assert(HL >= 1 && (HL & (HL - 1)) == 0 && HL <= kWave, "head must be 2^k lanes");
    static_assert(NW >= CPL, "one look-back wave per 64 channels of the block");
};

// Per-(dtype, Dh) launch configuration of the forward and backward scans.
// The forward runs 512-thread workgroups (8 waves): at 64K context a tile is then 256 steps
// (128 with one-byte storage), which halves the look-back words per byte of data against 256
// threads and measured ~7 % faster.  The backward holds more per thread (232 VGPRs, 2 waves
// per SIMD), so a 512-thread workgroup would leave one workgroup per CU; it keeps 256
// threads.  A thread takes four steps of VEC channels, at most 32 elements (more would spill
// the backward's registers).  One-byte storage also takes 8 channels per thread, 8 bytes per
// step: 16 channels over two steps (256-thread forward workgroups, three to a CU) measured 6 %
// (forward) and 13 % (backward) slower at 64K context, with twice the slot-scan and
// look-back work per element and 16-channel thread spans whose LDS accesses collide in banks.
//
// Variant V = 1 of the forward takes 256-thread workgroups (tiles of half the depth).  The
// host picks it from a measured table (fwd_tile_variant in the dispatcher) for the problem
// sizes where it ran faster; it is built for fp16 storage with Dh = 64, where it was measured.
template <typename T, int DH, int V = 0>
struct FwdCfg {
    static constexpr int NT = V == 0 ? 512 : 256;
    static constexpr int L = 4;
    using G = Geom<T, DH, L, NT>;
};
template <typename T, int DH>
constexpr bool kHasFwdVariant = std::is_same<T, _Float16>::value && DH == 64;
template <typename T, int DH>
struct BwdCfg {
    static constexpr int NT = 256;
    static constexpr int S0 = Geom<T, DH, 1, NT>::S;
    // four steps per thread (at least 64 steps per tile): deeper tiles halve the look-back
    // words against two steps per thread and measured ~3 % faster at 64K context, although
    // the 232 VGPRs then allow two waves per SIMD rather than three
    static constexpr int L = 4 * S0 >= kCkptChunk ? 4 : kCkptChunk / S0;
    using G = Geom<T, DH, L, NT>;
    // the backward tile must start on a checkpoint boundary
    static_assert(G::TT % kCkptChunk == 0, "backward tile must be a multiple of 64 steps");
};

// Workspace layout: [header 256 B][flag X words][flag Y words][internal checkpoint].
struct WsHeader {
    uint32_t epoch;  // device epoch of launches recorded into graphs (bit 29 set once used)
    uint32_t reserved[2];
    // 0, or the inclusive tag of the last launch whose look-back wait timed out (its results
    // that depend on the missing value are NaN); only waits of that launch give up on it
    uint32_t abort;
    uint32_t pad0[4];
    // look-back statistics, counted by the statistics instance only (kChainStats): 8 sets
    // (workgroup ID mod 8, i.e. one per XCD) of kStatWords counters, see LbStat
    uint32_t stats[8 * 5];
    uint32_t pad[16];
};
constexpr int kStatWordsOffset = 8;  // header word of stats[0]
// Counters of one statistics set: lanes whose neighbouring tile already showed its inclusive
// value; lanes that walked back; earlier tiles folded during walks; the longest walk (tiles
// folded plus the inclusive value that ended it); unproductive polls.
enum LbStat : int { kStatTook = 0, kStatWalked = 1, kStatFolded = 2, kStatMaxWalk = 3,
                    kStatPolls = 4, kStatWords = 5 };
constexpr uint32_t kHostEpochMask = 0x1fffffffu;  // host epochs: bit 29 clear
constexpr uint32_t kDeviceEpochBit = 0x20000000u;  // device epochs: bit 29 set
static_assert(sizeof(WsHeader) == 256, "header must be 256 bytes");

constexpr uint32_t kTagAgg = 1u;
constexpr uint32_t kTagInc = 2u;

struct FwdParams {
    const void* a;
    const void* v;
    const void* q;   // NULL: no readout (checkpoint-only pass)
    const float* e0;  // NULL: zero initial state
    void* y;          // NULL: no readout
    float* eT;
    float* ckpt;
    float* prod;      // non-NULL (state-only pass): product of every gate over T, per lane
    uint32_t* hdr;
    uint64_t* flagX;
    uint64_t* flagY;
    int64_t T;
    int64_t C;       // H * Dh
    int64_t nLanes;  // B * C
    int64_t nck;     // ceil(T / 64)
    uint32_t nCB;
    uint32_t nTiles;
    uint32_t epoch;  // tags of this call's look-back words (host epoch)
    const uint32_t* epochWord;  // non-NULL: read the epoch here instead (graph-recorded launch)
    uint32_t det;    // 0, or the block of the reproducible look-back (a power of two)
    uint32_t withhold;  // non-zero: launch the forced-timeout test instance (see launch_fwd)
    uint32_t stats;     // non-zero: launch the look-back statistics instance
    uint32_t variant;   // tile-shape variant of FwdCfg (0 default, 1 where kHasFwdVariant)
};

struct BwdParams {
    const void* a;
    const void* v;
    const void* q;
    const void* dy;
    const float* e0;
    const float* dET;
    const float* ckpt;
    void* da;   // da, dv, dq all NULL: only de0 is written (sequence-segment aggregate)
    void* dv;
    void* dq;
    float* de0;
    uint32_t* hdr;
    uint64_t* flagX;
    uint64_t* flagY;
    int64_t T;
    int64_t C;
    int64_t nLanes;
    int64_t nck;
    uint32_t nCB;
    uint32_t nTiles;
    uint32_t epoch;
    const uint32_t* epochWord;
    uint32_t det;
    uint32_t withhold;
    uint32_t stats;
};

struct StepParams {
    const void* a;
    const void* v;
    const void* q;
    float* state;
    void* y;
    int64_t nLanes;
};

// Host-visible launchers, explicitly instantiated in the kernel translation units.
template <typename T, int MODE, int DH>
hipError_t launch_fwd(const FwdParams& p, hipStream_t s);
template <typename T, int MODE, int DH>
hipError_t launch_bwd(const BwdParams& p, hipStream_t s);
template <typename T, int MODE, int DH>
hipError_t launch_step(const StepParams& p, hipStream_t s);
hipError_t launch_fill_zero(void* dst, size_t bytes, hipStream_t s);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t s);
hipError_t launch_fill_f32(float* dst, float value, int64_t n, hipStream_t s);
hipError_t launch_epoch_bump(uint32_t* word, hipStream_t s);
hipError_t launch_compose(int64_t nseg, int64_t nLanes, int reverse, const float* prod,
                          const float* agg, const float* boundary, float* carry, float* total,
                          hipStream_t s);

#if defined(__HIP_DEVICE_COMPILE__) || defined(__HIPCC__)

// ---------------------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------------------
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

// VEC values of storage (16 bytes; 8 bytes in x, y for one-byte storage) -> VEC fp32 values
// (exact).
template <typename T>
__device__ __forceinline__ void unpack(const uint4& r, float* out);
template <>
__device__ __forceinline__ void unpack<float>(const uint4& r, float* out) {
    out[0] = __uint_as_float(r.x);
    out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z);
    out[3] = __uint_as_float(r.w);
}
template <>
__device__ __forceinline__ void unpack<_Float16>(const uint4& r, float* out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        half2_t h = __builtin_bit_cast(half2_t, w[k]);
        out[2 * k] = (float)h.x;
        out[2 * k + 1] = (float)h.y;
    }
}
template <>
__device__ __forceinline__ void unpack<__bf16>(const uint4& r, float* out) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        out[2 * k] = __uint_as_float(w[k] << 16);
        out[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}

// One-byte formats: a thread's 8 values are the two words x, y; each holds four values, byte
// k = element k; the packed conversions take or fill the low (false) or high (true) 16-bit
// half of a word.
typedef float f2_t __attribute__((ext_vector_type(2)));
template <bool E5M2>
__device__ __forceinline__ void unpack_f8(const uint4& r, float* out) {
    const uint32_t w[2] = {r.x, r.y};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        f2_t lo, hi;
        if constexpr (E5M2) {
            lo = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[k], false);
            hi = __builtin_amdgcn_cvt_pk_f32_bf8((int)w[k], true);
        } else {
            lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], false);
            hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[k], true);
        }
        out[4 * k] = lo.x;
        out[4 * k + 1] = lo.y;
        out[4 * k + 2] = hi.x;
        out[4 * k + 3] = hi.y;
    }
}
template <>
__device__ __forceinline__ void unpack<f8e4m3>(const uint4& r, float* out) {
    unpack_f8<false>(r, out);
}
template <>
__device__ __forceinline__ void unpack<f8e5m2>(const uint4& r, float* out) {
    unpack_f8<true>(r, out);
}

// VEC fp32 values -> VEC values of storage (round to nearest even).
template <typename T>
__device__ __forceinline__ uint4 pack(const float* x);
template <>
__device__ __forceinline__ uint4 pack<float>(const float* x) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
}
template <>
__device__ __forceinline__ uint4 pack<_Float16>(const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        half2_t h = {(_Float16)x[2 * k], (_Float16)x[2 * k + 1]};
        w[k] = __builtin_bit_cast(uint32_t, h);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}
template <>
__device__ __forceinline__ uint4 pack<__bf16>(const float* x) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        bf2_t h = {(__bf16)x[2 * k], (__bf16)x[2 * k + 1]};
        w[k] = __builtin_bit_cast(uint32_t, h);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Out-of-range values follow the formats' own conversion: NaN for E4M3 beyond 464 in
// magnitude, infinity for E5M2 beyond 61440.  The first conversion of a word fills its low
// half and keeps the high half of its `old` operand, which the second one then overwrites:
// `old` is given the first input's bits rather than 0, which would cost a move per word.
template <bool E5M2>
__device__ __forceinline__ uint4 pack_f8(const float* x) {
    uint32_t w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        int v;
        const int any = __float_as_int(x[4 * k]);
        if constexpr (E5M2) {
            v = __builtin_amdgcn_cvt_pk_bf8_f32(x[4 * k], x[4 * k + 1], any, false);
            v = __builtin_amdgcn_cvt_pk_bf8_f32(x[4 * k + 2], x[4 * k + 3], v, true);
        } else {
            v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k], x[4 * k + 1], any, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * k + 2], x[4 * k + 3], v, true);
        }
        w[k] = (uint32_t)v;
    }
    return make_uint4(w[0], w[1], 0u, 0u);
}
template <>
__device__ __forceinline__ uint4 pack<f8e4m3>(const float* x) {
    return pack_f8<false>(x);
}
template <>
__device__ __forceinline__ uint4 pack<f8e5m2>(const float* x) {
    return pack_f8<true>(x);
}

// Raw buffer access for tiles that lie inside one batch row: a workgroup-uniform resource
// (base = the tile's first element in this channel block) in scalar registers, one 32-bit
// lane offset shared by every step, and the step's row offset as a scalar offset.  This
// replaces a 64-bit vector address per load or store.  Word 3 is the raw 32-bit-element
// format of gfx9-family buffer resources; the range check is never reached (offsets stay
// below 2^31 by construction).
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
constexpr int kBufWord3 = 0x00020000;
// Cache policy of the streaming accesses: non-temporal.  Every element is read once and
// written once, so nothing is kept for reuse; on MI355X this lifts a 3-read/1-write stream
// from about 5.7 to about 6.1 TB/s.
constexpr int kStreamPolicy = 2;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff,
                                             kBufWord3);
}
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ uint4 ldbuf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int32_t soff) {
    if constexpr (kVB<T> == 16) {
        const v4u_t x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, kStreamPolicy);
        return make_uint4(x.x, x.y, x.z, x.w);
    } else {
        const v2u_t x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, soff, kStreamPolicy);
        return make_uint4(x.x, x.y, 0u, 0u);
    }
}
// Stores take their row offset in the resource base and a constant scalar offset of 0.  A
// 16-byte buffer store that names a scalar-register offset gets no wait state before the
// next instruction overwrites its data registers, and on gfx950 the store can then write
// the new value for some lanes (seen as corrupted dq rows); with a constant offset the
// compiler keeps the required gap.
template <typename T>
__device__ __forceinline__ void stbuf(const void* row_base, uint32_t voff, const uint4& v) {
    if constexpr (kVB<T> == 16) {
        const v4u_t x = {v.x, v.y, v.z, v.w};
        __builtin_amdgcn_raw_buffer_store_b128(x, make_rsrc(row_base), (int)voff, 0, kStreamPolicy);
    } else {
        const v2u_t x = {v.x, v.y};
        __builtin_amdgcn_raw_buffer_store_b64(x, make_rsrc(row_base), (int)voff, 0, kStreamPolicy);
    }
}
template <typename T>
__device__ __forceinline__ uint4 ld16(const void* base, int64_t elem_off, int esize) {
    const char* p = static_cast<const char*>(base) + elem_off * esize;
    if constexpr (kVB<T> == 16) {
        return *reinterpret_cast<const uint4*>(p);
    } else {
        const uint2 x = *reinterpret_cast<const uint2*>(p);
        return make_uint4(x.x, x.y, 0u, 0u);
    }
}
template <typename T>
__device__ __forceinline__ void st16(void* base, int64_t elem_off, int esize, const uint4& v) {
    char* p = static_cast<char*>(base) + elem_off * esize;
    if constexpr (kVB<T> == 16)
        *reinterpret_cast<uint4*>(p) = v;
    else
        *reinterpret_cast<uint2*>(p) = make_uint2(v.x, v.y);
}

// Gate complement: u = 1 - s = sigma(-a) = 1 / (1 + exp(a)), for s = sigma(a).  The kernels
// carry gates only as complements (see GP and update()), so s itself is never formed.  u
// keeps its full relative precision where s is close to 1 (long memory), which 1 - s computed
// by subtraction would lose.  No clamp is needed: for a above about 88, exp(a) is +inf and u
// is 0 (s = 1); for a below about -104, exp(a) is 0 and u is 1 (s = 0); a NaN logit gives NaN.
// The backward's gate derivative s (1 - s) = u - u^2 is taken from u with one fma: exact
// relative to u, and within one unit in the last place of u absolutely (so relatively coarse
// only where s itself is tiny, where the derivative is small against its neighbours; the
// 16- and 8-bit bars are far wider than that error, fp32 storage uses gate_u_slope).
__device__ __forceinline__ float gate_u(float a) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * 1.4426950408889634f));
}
__device__ __forceinline__ float gate_slope(float u) { return __builtin_fmaf(-u, u, u); }

// One-byte storage has only 256 logit codes: the scans evaluate gate_u once per code into a
// table in LDS at the start of a workgroup and look every step's complement up there, one
// byte extraction and one LDS read in place of the decode, exponential, add and reciprocal.
// The table holds gate_u of the decoded code, so the values are the same bits as evaluated
// in place.
template <typename T>
constexpr bool kGateTable = sizeof(T) == 1;
template <typename T, int NT>
__device__ __forceinline__ void fill_gate_table(float* tab) {
    for (int i = threadIdx.x; i < 256; i += NT) {
        float a[Storage<T>::VEC];
        unpack<T>(make_uint4((uint32_t)i, 0u, 0u, 0u), a);
        tab[i] = gate_u(a[0]);
    }
}
// The complements of a thread's 8 one-byte logits (words x, y; byte k = element k).
__device__ __forceinline__ void gate_u_lookup(const uint4& r, const float* tab, float* u) {
    const uint32_t w[2] = {r.x, r.y};
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) u[4 * k + e] = tab[(w[k] >> (8 * e)) & 0xffu];
}
// The same complement with the derivative s (1 - s) = exp(a) u^2 to full relative precision,
// for fp32 storage, whose bar would see the absolute error of u - u^2 where s is small.
// exp(a) is capped at 2^126 so that s (1 - s) is 0, not NaN, where it overflows (u is 0
// there).
__device__ __forceinline__ float gate_u_slope(float a, float& slope) {
    const float e = __builtin_amdgcn_exp2f(a * 1.4426950408889634f);
    const float u = __builtin_amdgcn_rcpf(1.0f + e);
    slope = __builtin_fminf(e, 0x1p126f) * u * u;
    return u;
}

// a * b + c rounded once, in the operands' own type.
__device__ __forceinline__ float fma_(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_(double a, double b, double c) { return __builtin_fma(a, b, c); }

// One step of the recurrence on the state x: x' = s x + b with s = 1 - u, b = u v (controlled)
// or v (direct), one fma on x.  s = 1 - u is exact for u >= 1/2 and otherwise rounds by at
// most 2^-25 (unbiased), i.e. one rounding relative to x as in any update; u itself (the
// complement, relatively exact) is what the gate products use (see GP).  A masked step passes
// s = 1, b = 0, which leaves x unchanged.
template <int MODE, typename F>
__device__ __forceinline__ F step_b(F u, F v) {
    if constexpr (MODE == kControlled) return u * v;
    else return v;
}
template <typename F>
__device__ __forceinline__ F update(F x, F s, F b) { return fma_(s, x, b); }

// The type the scans accumulate in: fp64 for fp32 storage, fp32 otherwise.  fp32 storage has
// the tightest bar (1e-5) and long-memory lanes sum thousands of roundings of the state and
// of its reverse-time gradient, which fp32 accumulation leaves at about that size (a
// sequential fp32 loop misses the bar there too).  On gfx950 a non-packed fp32 fma and an
// fp64 fma issue at the same rate, so accumulating in fp64 costs registers, LDS and
// conversions rather than issue slots; the 16- and 8-bit kernels, whose bars are 500 times
// wider, keep fp32.  Gates, readout and look-back words stay fp32.
template <typename T>
using Acc = typename std::conditional<sizeof(T) == 4, double, float>::type;

// Sum over the HL consecutive, aligned threads that hold one head; every thread of the head
// receives the total.  Up to 16 threads (one DPP row) the butterfly uses DPP lane moves:
// swap neighbours, swap pairs, mirror each half row, mirror the row.  Wider heads use
// cross-row shuffles.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int HL>
__device__ __forceinline__ float head_sum(float x) {
    if constexpr (HL >= 2) x = dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (HL >= 4) x = dpp_add<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (HL >= 8) x = dpp_add<0x141>(x);  // row_half_mirror
    if constexpr (HL >= 16) x = dpp_add<0x140>(x); // row_mirror
#pragma unroll
    for (int m = 16; m < HL; m <<= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// Gate products of a pair, in one of two representations.  GP<true>, used by every scan, carries
// the complement q = 1 - P of a product P of gates: along a long-memory lane the gates lie
// within 1e-4 of 1, and an fp32 product of two such factors drops its second-order term
// (below half a unit in the last place next to 1), always in the same direction; the
// cross-tile carry c <- e + P c divides that bias by 1 - P, so the state would drift along
// the sequence.  The complement of a product, q1 + q2 - q1 q2, keeps its relative precision,
// and (1 - q) x = x - q x loses nothing next to 1.  Where P is small instead, the complement
// leaves an absolute error of about one unit in the last place of x in (1 - q) x, i.e.
// relative to the state being decayed, which the parity metric's scale already covers.
// GP<false> carries the product itself: the plain form of the same interface.
template <bool CQ, typename F = float>
struct GP;
//
// Operations (p, q: products in the representation; x, e: states):
//   mul(a, b)      the product of two gate products
//   apply(p, x)    p x
//   comp(p, x, e)  e + p x, the pair combine's state part
// For complements, mul is q1 + q2 - q1 q2 = q1 (1 - q2) + q2 and comp is (1 - q) x + e, each
// one fma on the running value a or x, after a subtraction that does not depend on it (so a
// serial fold is one dependent fma per step).  1 - q is exact for q >= 1/2 and rounds by at
// most 2^-25 below; that error is multiplied by a <= 1 (relative to the result, at most
// 2^-25) or by x (relative to x, as any rounding of the state), and it is unbiased, unlike the
// product of two near-one factors.
template <typename F>
struct GP<false, F> {
    static constexpr F one = F(1);
    __device__ static __forceinline__ F mul(F a, F b) { return a * b; }
    __device__ static __forceinline__ F apply(F p, F x) { return p * x; }
    __device__ static __forceinline__ F comp(F p, F x, F e) { return fma_(p, x, e); }
};
template <typename F>
struct GP<true, F> {
    static constexpr F one = F(0);
    __device__ static __forceinline__ F mul(F a, F b) { return fma_(a, F(1) - b, b); }
    __device__ static __forceinline__ F apply(F q, F x) { return fma_(-q, x, x); }
    __device__ static __forceinline__ F comp(F q, F x, F e) { return fma_(F(1) - q, x, e); }
};

// Exclusive scan of the per-thread pairs over the S time slots of a tile, per channel, in
// two phases through LDS (thread = slot * NCL + channel lane, VEC channels each; the slots
// of wave w are w*SPW .. w*SPW+SPW-1).
//
// Phase A: every thread stores its pair; lane = channel of each wave then walks that wave's
// SPW slots in order (backwards for the reverse scan), keeps each slot's exclusive pair within
// the wave in registers, and stores the wave's aggregate.  No barrier is needed inside phase
// A: a wave only reads what it has just written, and LDS serves one wave's requests in order.
// Phase B (after a barrier): lane = channel composes the other waves' aggregates into the
// wave prefix and stores each slot's exclusive pair for the whole tile.
// Forward pairs compose earlier first, (P1, E1) o (P2, E2) = (P1 P2, E2 + P2 E1); reverse
// maps lam_out = P lam_in + E compose the later side first; both reduce to the same update
// (te, tp) <- (p te + e, tp p) in their own walking order, with the products in GP<CQ>'s
// representation.
// N consecutive values between registers and LDS in 16-byte pieces (the address is 16-byte
// aligned: a thread's VEC channels of one slot row).
template <int N>
__device__ __forceinline__ void lds_store(float* dst, const float* x) {
#pragma unroll
    for (int e = 0; e < N; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(x[e], x[e + 1], x[e + 2], x[e + 3]);
}
template <int N>
__device__ __forceinline__ void lds_store(double* dst, const double* x) {
#pragma unroll
    for (int e = 0; e < N; e += 2) *reinterpret_cast<double2*>(dst + e) = make_double2(x[e], x[e + 1]);
}
template <int N>
__device__ __forceinline__ void lds_load(const float* src, float* x) {
#pragma unroll
    for (int e = 0; e < N; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(src + e);
        x[e] = v.x;
        x[e + 1] = v.y;
        x[e + 2] = v.z;
        x[e + 3] = v.w;
    }
}
template <int N>
__device__ __forceinline__ void lds_load(const double* src, double* x) {
#pragma unroll
    for (int e = 0; e < N; e += 2) {
        const double2 v = *reinterpret_cast<const double2*>(src + e);
        x[e] = v.x;
        x[e + 1] = v.y;
    }
}

template <class G, bool REV, bool CQ, typename F>
__device__ __forceinline__ void slots_phase_a(const F* P, const F* E, F* sP, F* sE, F* sWP, F* sWE,
                                              F (&xp)[G::CPL][G::SPW], F (&xe)[G::CPL][G::SPW]) {
    constexpr int VEC = G::VEC, CB = G::CB, NCL = G::NCL, SPW = G::SPW;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
    const int j = tid % NCL, slot = tid / NCL;
    lds_store<VEC>(sP + slot * CB + j * VEC, P);
    lds_store<VEC>(sE + slot * CB + j * VEC, E);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int k = 0; k < G::CPL; ++k) {
        const int ch = lane + k * kWave;
        F tp = GP<CQ, F>::one, te = F(0);
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int sw = REV ? SPW - 1 - q : q;
            const int s = w * SPW + sw;
            const F ps = sP[s * CB + ch], es = sE[s * CB + ch];
            xp[k][sw] = tp;
            xe[k][sw] = te;
            te = GP<CQ, F>::comp(ps, te, es);
            tp = GP<CQ, F>::mul(tp, ps);
        }
        sWP[w * CB + ch] = tp;
        sWE[w * CB + ch] = te;
    }
}

template <class G, bool REV, bool CQ, typename F>
__device__ __forceinline__ void slots_phase_b(F* sP, F* sE, const F* sWP, const F* sWE,
                                              const F (&xp)[G::CPL][G::SPW],
                                              const F (&xe)[G::CPL][G::SPW]) {
    constexpr int CB = G::CB, SPW = G::SPW, NW = G::NW;
    const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
#pragma unroll
    for (int k = 0; k < G::CPL; ++k) {
        const int ch = lane + k * kWave;
        F wp = GP<CQ, F>::one, we = F(0);  // the other waves on this slot's earlier side
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            const int v = REV ? NW - 1 - q : q;
            if (REV ? v > w : v < w) {
                const F pv = sWP[v * CB + ch], ev = sWE[v * CB + ch];
                we = GP<CQ, F>::comp(pv, we, ev);
                wp = GP<CQ, F>::mul(wp, pv);
            }
        }
#pragma unroll
        for (int sw = 0; sw < SPW; ++sw) {
            const int s = w * SPW + sw;
            sP[s * CB + ch] = GP<CQ, F>::mul(xp[k][sw], wp);
            sE[s * CB + ch] = GP<CQ, F>::comp(xp[k][sw], we, xe[k][sw]);
        }
    }
}

// Composition of all waves' aggregates for channel ch: the tile's own pair / map.
template <class G, bool REV, bool CQ, typename F>
__device__ __forceinline__ void tile_total(const F* sWP, const F* sWE, int ch, F& tp, F& te) {
    tp = GP<CQ, F>::one;
    te = F(0);
#pragma unroll
    for (int q = 0; q < G::NW; ++q) {
        const int v = REV ? G::NW - 1 - q : q;
        const F pv = sWP[v * G::CB + ch], ev = sWE[v * G::CB + ch];
        te = GP<CQ, F>::comp(pv, te, ev);
        tp = GP<CQ, F>::mul(tp, pv);
    }
}

// The tile-wide exclusive pair of this thread's slot, for its VEC channels.
template <class G, typename F>
__device__ __forceinline__ void read_exclusive(const F* sP, const F* sE, F* XP, F* XE) {
    const int j = threadIdx.x % G::NCL, slot = threadIdx.x / G::NCL;
    lds_load<G::VEC>(sP + slot * G::CB + j * G::VEC, XP);
    lds_load<G::VEC>(sE + slot * G::CB + j * G::VEC, XE);
}

__device__ __forceinline__ uint64_t tag_word(uint32_t tag, float v) {
    return (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(__float_as_uint(v));
}
__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, float v) {
    __hip_atomic_store(p, tag_word(tag, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return static_cast<uint32_t>(w >> 32); }
__device__ __forceinline__ float word_val(uint64_t w) {
    return __uint_as_float(static_cast<uint32_t>(w));
}

// Decoupled look-back over one channel's chain of tiles.  `step` is -1 (walk toward earlier
// tiles, forward scan) or +1 (toward later tiles, reverse scan).  Returns the carry entering
// tile `tile`: the composition of the published pairs, ended by an inclusive value.
//
// The wait is bounded: after LIMIT polls without progress (kSpinLimit; kTestSpinLimit in the
// forced-timeout test instances) the workgroup raises the
// sticky abort word of the workspace header and returns NaN, and every other waiting
// workgroup that sees the abort word returns NaN too, so a broken chain drains instead of
// hanging.  A correct run never comes near the limit (about a second of polling).
//
// With PROD (sequence-segment aggregates) a tile's inclusive word in flagY holds the product
// of every gate from the chain's start through that tile (in GP<CQ>'s representation);
// *pinc then receives the product through the tile before `tile` (NaN when the wait gave
// up).
constexpr uint32_t kSpinLimit = 1u << 20;
// The forced-timeout test instances (a separate kernel instantiation, so the normal kernels
// carry no trace of it): the chain's first tile withholds its publications and every wait
// gives up after kTestSpinLimit polls.
constexpr uint32_t kTestSpinLimit = 4096;

// One unproductive poll of a bounded wait: false once the wait must give up (this launch's
// tag is in the abort word, or this wait has polled LIMIT times; then it puts it there).  The
// abort word holds the tag of the launch that timed out, so a timeout never makes the waits
// of later launches on the same workspace give up.
template <uint32_t LIMIT = kSpinLimit>
__device__ __forceinline__ bool wait_turn(uint32_t polls, uint32_t* hdr, uint32_t abortTag) {
    if ((polls & 255u) == 0u) {
        const bool abort = __hip_atomic_load(&hdr[3], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) == abortTag;
        if (abort || polls >= LIMIT) {
            if (!abort)
                __hip_atomic_store(&hdr[3], abortTag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// What one lane's walk did, for the statistics instance: earlier tiles folded, unproductive
// polls.
struct WalkCount {
    uint32_t folded;
    uint32_t polls;
};

//
// F is the type the walk folds the published fp32 values in: the kernel's accumulation type
// (Acc), so that a long walk adds no roundings of its own in the fp64-accumulating kernels.
template <bool PROD = false, uint32_t LIMIT = kSpinLimit, bool CQ = false, typename F = float>
__device__ __forceinline__ F look_back(const uint64_t* flagX, const uint64_t* flagY,
                                       int64_t nLanes, int64_t lane, int64_t tile, int step,
                                       uint32_t tagAgg, uint32_t tagInc, uint32_t* hdr,
                                       float* pinc = nullptr, WalkCount* wc = nullptr) {
    using Q = GP<CQ, F>;
    F ap = Q::one, ae = F(0);
    int64_t j = tile + step;
    uint32_t polls = 0;
    for (;;) {
        // both words of the slot in one round trip
        const uint64_t x = peek(flagX + j * nLanes + lane);
        const uint64_t yv = peek(flagY + j * nLanes + lane);
        const uint32_t tg = word_tag(x);
        if (tg == tagInc) {
            if constexpr (!PROD) {
                if (wc) *wc = WalkCount{(uint32_t)((j - tile) * step - 1), polls};
                return Q::comp(ap, F(word_val(x)), ae);
            }
            // the inclusive product is published beside the inclusive state, in no fixed
            // order: wait until it is visible too
            if (word_tag(yv) == tagInc) {
                *pinc = float(Q::mul(ap, F(word_val(yv))));
                return Q::comp(ap, F(word_val(x)), ae);
            }
        }
        if (tg == tagAgg && word_tag(yv) == tagAgg) {
            ae = Q::comp(ap, F(word_val(x)), ae);
            ap = Q::mul(ap, F(word_val(yv)));
            j += step;
            continue;
        }
        if (!wait_turn<LIMIT>(++polls, hdr, tagInc)) {
            if constexpr (PROD) *pinc = __builtin_nanf("");
            if (wc) *wc = WalkCount{(uint32_t)((j - tile) * step - 1), polls};
            return F(__builtin_nanf(""));
        }
    }
}

// Look-back variants, one kernel instance each, so the default kernels carry no code of the
// others: the default look-back; the reproducible one (ESA_DETERMINISTIC); the forced-timeout
// test instance (either look-back, chosen at run time, with the chain's first tile withholding
// its publications and every wait giving up after kTestSpinLimit polls).
// The statistics instance (kChainStats) is the default look-back with counters (LbStat).
enum : int { kChainDefault = 0, kChainDet = 1, kChainTest = 2, kChainStats = 3 };

// The carry entering `tile` on one lane's chain.  When the neighbouring tile on the earlier
// side has already published its inclusive value -- the usual case once a chain's earlier
// tiles were dispatched well before this one -- the tile takes it directly and publishes no
// aggregate pair, so its only look-back traffic is its own inclusive word (8 instead of 24
// bytes per lane; measured 0.6-2.3 % faster at 64K context).  Otherwise it publishes its
// aggregate pair (te, tp) and walks back.  The caller then publishes the inclusive value.
// Successors cope with a tile that never publishes an aggregate: they wait for its
// inclusive word, which follows without any wait of its own.
//
// With `det` = K (a power of two) the chain is cut into blocks of K tiles, counted from its
// start, and only the chain's first tile and the last tile of each block publish inclusive
// values; the others publish their aggregate pair and nothing else (det_publishes_inc).
// Every word slot then only ever holds one kind of word, so the walk below folds exactly the
// aggregates back to the nearest publisher and ends at its inclusive value: the carry is the
// same fp32 expression on every run (bitwise reproducible results), whatever the timing.
// With K = 1 every tile waits for its neighbour's inclusive value.  The host picks K from the
// number of chains, so that a block's walk stays short while the inclusive values still move
// K tiles per hop.
template <bool PROD = false, uint32_t LIMIT = kSpinLimit, bool CQ = false, typename F = float>
__device__ __forceinline__ F chain_carry(uint64_t* flagX, uint64_t* flagY, int64_t nLanes,
                                         int64_t lane, int64_t tile, int step, uint32_t tagAgg,
                                         uint32_t tagInc, uint32_t* hdr, float tp, float te,
                                         float* pin, uint32_t det, bool pubInc,
                                         WalkCount* wc = nullptr) {
    if (det == 0u) {
        const uint64_t x = peek(flagX + (tile + step) * nLanes + lane);
        if (word_tag(x) == tagInc) {
            if constexpr (!PROD) return F(word_val(x));
            const uint64_t y = peek(flagY + (tile + step) * nLanes + lane);
            if (word_tag(y) == tagInc) {
                *pin = word_val(y);
                return F(word_val(x));
            }
        }
    }
    if (det == 0u || !pubInc) {
        publish(flagX + tile * nLanes + lane, tagAgg, te);
        publish(flagY + tile * nLanes + lane, tagAgg, tp);
    }
    if (wc) *wc = WalkCount{0u, 0u};
    return look_back<PROD, LIMIT, CQ, F>(flagX, flagY, nLanes, lane, tile, step, tagAgg, tagInc,
                                         hdr, pin, wc);
}

// Statistics instance: adds this wave's look-back outcome to the workgroup's set of counters
// (one set per XCD, by workgroup ID), one atomic per counter and wave.  `walked` lanes
// returned a WalkCount; the others took their neighbour's inclusive value directly.
__device__ __forceinline__ void count_walks(uint32_t* hdr, bool active, bool walked,
                                            const WalkCount& wc) {
    const uint64_t act = __ballot(active);
    const uint64_t wlk = __ballot(active && walked);
    uint32_t folded = active && walked ? wc.folded : 0u;
    uint32_t polls = active && walked ? wc.polls : 0u;
    uint32_t longest = active && walked ? wc.folded + 1u : 0u;
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) {
        folded += __shfl_xor(folded, m, kWave);
        polls += __shfl_xor(polls, m, kWave);
        const uint32_t o = __shfl_xor(longest, m, kWave);
        longest = o > longest ? o : longest;
    }
    if ((threadIdx.x % kWave) == 0) {
        uint32_t* st = hdr + kStatWordsOffset + (blockIdx.x & 7u) * kStatWords;
        const uint32_t took = (uint32_t)__popcll(act & ~wlk), walk = (uint32_t)__popcll(wlk);
        __hip_atomic_fetch_add(st + kStatTook, took, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(st + kStatWalked, walk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(st + kStatFolded, folded, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(st + kStatMaxWalk, longest, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(st + kStatPolls, polls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Whether the tile at position `pos` along its chain (0 = the chain's first tile) publishes
// its inclusive value under `det` (see chain_carry).
__device__ __forceinline__ bool det_publishes_inc(uint32_t pos, uint32_t det) {
    return det == 0u || pos == 0u || (pos & (det - 1u)) == det - 1u;
}

// Workgroup -> (tile row, channel block).  Workgroup i runs on XCD i mod 8.  When the channel
// blocks split evenly over the 8 XCDs, XCD x owns the contiguous channel blocks
// [x nCB/8, (x+1) nCB/8) -- whole rows of the [B, T, H, Dh] tensors -- and walks them tile row
// by tile row, so the 128-byte pieces of one row that neighbouring workgroups read reach
// memory from one XCD, and each look-back chain stays inside one XCD.  Otherwise the order
// is plain tile-major.  Either way a tile's predecessor in its chain has a smaller workgroup
// ID, which is all the progress argument needs, whatever the real XCD placement.
__device__ __forceinline__ void tile_of(uint32_t wg, uint32_t nCB, uint32_t& row, uint32_t& cb) {
    if ((nCB & 7u) == 0u) {
        const uint32_t x = wg & 7u, m = wg >> 3, nx = nCB >> 3;
        row = m / nx;
        cb = x * nx + (m - row * nx);
    } else {
        row = wg / nCB;
        cb = wg - row * nCB;
    }
}

__device__ __forceinline__ uint32_t make_tag(uint32_t epoch, uint32_t kind) {
    return (epoch << 2) | kind;
}

// The epoch of this launch: the host's, or the workspace's device epoch for a launch recorded
// into a graph (advanced by epoch_bump_kernel before every replay of the launch).
__device__ __forceinline__ uint32_t launch_epoch(uint32_t host_epoch, const uint32_t* word) {
    return word ? __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : host_epoch;
}

#endif  // device compile

}  // namespace esa
