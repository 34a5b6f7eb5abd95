// Host side of libesa.so: argument validation, workspace layout and kernel dispatch over
// (dtype, mode, Dh).  Every check runs before the first HIP call, so an invalid call
// changes nothing on the device.  The library allocates nothing and never synchronises.
#include <stdint.h>
#include <string.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "esa.h"
#include "esa_common.hpp"

using namespace esa;

namespace {

struct Problem {
    int64_t B, T, H, Dh, C, nLanes, nElem;
    int dtype, mode;  // mode: the recurrence form (ESA_DIRECT / ESA_CONTROLLED)
    uint32_t det;     // ESA_DETERMINISTIC was set
    uint32_t forceTimeout;  // ESA_TEST_FORCE_TIMEOUT was set
    uint32_t stats;   // ESA_LOOKBACK_STATS was set
    int64_t esize;
};

struct TileShape {
    int CB, TTf, TTb;
    int TTf1;  // tile length of forward variant 1, or 0 where it is not built
};

template <typename T, int DH>
TileShape tile_shape_of() {
    return TileShape{FwdCfg<T, DH>::G::CB, FwdCfg<T, DH>::G::TT, BwdCfg<T, DH>::G::TT,
                     kHasFwdVariant<T, DH> ? FwdCfg<T, DH, 1>::G::TT : 0};
}

template <typename T>
TileShape tile_shape_dh(int64_t Dh) {
    switch (Dh) {
        case 16: return tile_shape_of<T, 16>();
        case 32: return tile_shape_of<T, 32>();
        case 64: return tile_shape_of<T, 64>();
        default: return tile_shape_of<T, 128>();
    }
}

TileShape tile_shape(int dtype, int64_t Dh) {
    switch (dtype) {
        case ESA_F32: return tile_shape_dh<float>(Dh);
        case ESA_F16: return tile_shape_dh<_Float16>(Dh);
        case ESA_BF16: return tile_shape_dh<__bf16>(Dh);
        case ESA_F8E4M3: return tile_shape_dh<f8e4m3>(Dh);
        default: return tile_shape_dh<f8e5m2>(Dh);
    }
}

int64_t storage_bytes(int dtype) {
    switch (dtype) {
        case ESA_F32: return 4;
        case ESA_F16:
        case ESA_BF16: return 2;
        default: return 1;
    }
}

bool supported_dh(int64_t Dh) { return Dh == 16 || Dh == 32 || Dh == 64 || Dh == 128; }

bool mul64(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_sizes(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode, Problem* pr) {
    const int form = mode & ~(ESA_DETERMINISTIC | ESA_TEST_FORCE_TIMEOUT | ESA_LOOKBACK_STATS);
    if (dtype < ESA_F32 || dtype > ESA_F8E5M2 || form < ESA_DIRECT || form > ESA_CONTROLLED)
        return ESA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Dh < 1 || T < 0) return ESA_ERR_INVALID_ARG;
    if (!supported_dh(Dh)) return ESA_ERR_UNSUPPORTED;
    pr->B = B;
    pr->T = T;
    pr->H = H;
    pr->Dh = Dh;
    pr->dtype = dtype;
    pr->mode = form;
    pr->det = (mode & ESA_DETERMINISTIC) ? 1u : 0u;
    pr->forceTimeout = (mode & ESA_TEST_FORCE_TIMEOUT) ? 1u : 0u;
    pr->stats = (mode & ESA_LOOKBACK_STATS) ? 1u : 0u;
    pr->esize = storage_bytes(dtype);
    int64_t bytes;
    if (!mul64(H, Dh, &pr->C) || !mul64(B, pr->C, &pr->nLanes) || !mul64(pr->nLanes, T, &pr->nElem) ||
        !mul64(pr->nElem, 4, &bytes) || !mul64(pr->nLanes, 16, &bytes))
        return ESA_ERR_INVALID_ARG;
    return ESA_OK;
}

// ESA_TEST_FORCE_TIMEOUT is accepted by the readout forward and the gradient backward, for
// fp16 storage and Dh = 64 (the problems with a test instance of the kernels).
//
// ESA_LOOKBACK_STATS likewise, for fp16 and fp8 E4M3 storage with Dh = 64; it cannot be
// combined with ESA_DETERMINISTIC or ESA_TEST_FORCE_TIMEOUT (the statistics count the
// default look-back).
int check_test_flag(const Problem& pr, bool call_allows_it) {
    if (pr.stats) {
        if (!call_allows_it || pr.det || pr.forceTimeout) return ESA_ERR_INVALID_ARG;
        if (!((pr.dtype == ESA_F16 || pr.dtype == ESA_F8E4M3) && pr.Dh == 64))
            return ESA_ERR_UNSUPPORTED;
    }
    if (!pr.forceTimeout) return ESA_OK;
    if (!call_allows_it) return ESA_ERR_INVALID_ARG;
    return pr.dtype == ESA_F16 && pr.Dh == 64 ? ESA_OK : ESA_ERR_UNSUPPORTED;
}

struct Layout {
    uint32_t nCB, nTilesF, nTilesB;
    uint32_t fwdVariant, nTilesFV;  // the readout forward's tile-shape variant and its tiles
    int64_t nck;
    size_t offX, offY, offCk, total;
};

// The readout forward's tile-shape table (fp16 storage, Dh = 64, the default look-back): the
// problem classes -- the powers of two at or above the channel-block count and the sequence
// length -- where the 256-thread forward (128-step tiles, FwdCfg variant 1) ran faster than
// the 512-thread one (256-step tiles), by 4-10 %, in A/B sweeps of both on two boxes over
// 1-256 batch rows of 512 channels and 512-65536 steps.  Everything else, the 64K-context
// workload included, takes the 512-thread forward.  Chosen from the sizes alone, so a problem
// always runs the same kernels.
struct FwdTileClass {
    uint8_t lgCB, lgT;
};
constexpr FwdTileClass kFwd256[] = {{3, 9},  {3, 10},  {3, 11},  {5, 9},  {5, 10},
                                    {8, 14}, {9, 10},  {9, 11},  {9, 13}, {9, 14},
                                    {10, 12}, {10, 13}, {11, 9}, {11, 11}};

int ceil_log2(int64_t x) {
    int k = 0;
    while (k < 62 && (int64_t(1) << k) < x) ++k;
    return k;
}

uint32_t fwd_tile_variant(const Problem& pr, int64_t nCB) {
    if (pr.dtype != ESA_F16 || pr.Dh != 64 || pr.forceTimeout || pr.stats) return 0;
    const int lc = ceil_log2(nCB), lt = ceil_log2(pr.T);
    for (const FwdTileClass& c : kFwd256)
        if (c.lgCB == lc && c.lgT == lt) return 1;
    return 0;
}

// Workspace: [header 256 B][X words: nTiles x nLanes x 8 B][Y words: same][checkpoint].
int layout_of(const Problem& pr, Layout* L) {
    const TileShape ts = tile_shape(pr.dtype, pr.Dh);
    const int64_t nCB = cdiv(pr.nLanes, ts.CB);
    const uint32_t var = ts.TTf1 ? fwd_tile_variant(pr, nCB) : 0;
    const int64_t nTF = pr.T > 0 ? cdiv(pr.T, ts.TTf) : 0;
    const int64_t nTFV = var ? (pr.T > 0 ? cdiv(pr.T, ts.TTf1) : 0) : nTF;
    const int64_t nTB = pr.T > 0 ? cdiv(pr.T, ts.TTb) : 0;
    int64_t nTM = nTF > nTB ? nTF : nTB;
    nTM = nTFV > nTM ? nTFV : nTM;
    int64_t nwg, words, xbytes, ckbytes;
    if (!mul64(nCB, nTM, &nwg) || nwg > (int64_t)INT32_MAX)
        return ESA_ERR_UNSUPPORTED;
    if (!mul64(nTM, pr.nLanes, &words) || !mul64(words, 8, &xbytes)) return ESA_ERR_UNSUPPORTED;
    L->nCB = (uint32_t)nCB;
    L->nTilesF = (uint32_t)nTF;
    L->nTilesB = (uint32_t)nTB;
    L->fwdVariant = var;
    L->nTilesFV = (uint32_t)nTFV;
    L->nck = cdiv(pr.T, kCkptChunk);
    if (!mul64(L->nck, pr.nLanes, &ckbytes) || !mul64(ckbytes, 4, &ckbytes)) return ESA_ERR_UNSUPPORTED;
    L->offX = 256;
    L->offY = L->offX + align256((size_t)xbytes);
    L->offCk = L->offY + align256((size_t)xbytes);
    L->total = L->offCk + align256((size_t)ckbytes);
    return ESA_OK;
}

// The block of the reproducible look-back (0 without ESA_DETERMINISTIC): the smallest power
// of two K with K x (chains of the launch) >= kDetBlockTarget, at most kDetMaxBlock.  Few
// chains need long blocks, or their inclusive values, one hop per block, fall behind the
// workgroups in flight; long blocks lengthen every tile's walk over its block's aggregates.
// This rule was the fastest measured from 1 to 512 chains (fp16, bf16, fp32 and fp8).  It
// depends on the sizes and the storage type only, so a problem's results are the same on
// every run.
constexpr uint64_t kDetBlockTarget = 64;
constexpr uint32_t kDetMaxBlock = 16;
uint32_t det_block(const Problem& pr, uint32_t nCB) {
    if (!pr.det) return 0;
    uint32_t k = 1;
    while (k < kDetMaxBlock && (uint64_t)nCB * k < kDetBlockTarget) k <<= 1;
    return k;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
    const void* p;
    size_t n;
};

bool overlap(const Range& x, const Range& y) {
    if (!x.p || !y.p || x.n == 0 || y.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x.p), b0 = reinterpret_cast<uintptr_t>(y.p);
    return a0 < b0 + y.n && b0 < a0 + x.n;
}

// true if any output overlaps any input or another output
bool any_overlap(const Range* in, int nin, const Range* out, int nout) {
    for (int i = 0; i < nout; ++i) {
        for (int k = 0; k < nin; ++k)
            if (overlap(out[i], in[k])) return true;
        for (int k = i + 1; k < nout; ++k)
            if (overlap(out[i], out[k])) return true;
    }
    return false;
}

#define ESA_DISPATCH(KIND, dtype, mode, Dh, params, stream)                                   \
    [&]() -> hipError_t {                                                                     \
        switch (dtype * 2 + mode) {                                                           \
            case ESA_F32 * 2 + 0: return KIND##_dh<float, 0>(Dh, params, stream);            \
            case ESA_F32 * 2 + 1: return KIND##_dh<float, 1>(Dh, params, stream);            \
            case ESA_F16 * 2 + 0: return KIND##_dh<_Float16, 0>(Dh, params, stream);         \
            case ESA_F16 * 2 + 1: return KIND##_dh<_Float16, 1>(Dh, params, stream);         \
            case ESA_BF16 * 2 + 0: return KIND##_dh<__bf16, 0>(Dh, params, stream);          \
            case ESA_BF16 * 2 + 1: return KIND##_dh<__bf16, 1>(Dh, params, stream);          \
            case ESA_F8E4M3 * 2 + 0: return KIND##_dh<f8e4m3, 0>(Dh, params, stream);        \
            case ESA_F8E4M3 * 2 + 1: return KIND##_dh<f8e4m3, 1>(Dh, params, stream);        \
            case ESA_F8E5M2 * 2 + 0: return KIND##_dh<f8e5m2, 0>(Dh, params, stream);        \
            default: return KIND##_dh<f8e5m2, 1>(Dh, params, stream);                        \
        }                                                                                     \
    }()

template <typename T, int M>
hipError_t fwd_dh(int64_t Dh, const FwdParams& p, hipStream_t s) {
    switch (Dh) {
        case 16: return launch_fwd<T, M, 16>(p, s);
        case 32: return launch_fwd<T, M, 32>(p, s);
        case 64: return launch_fwd<T, M, 64>(p, s);
        default: return launch_fwd<T, M, 128>(p, s);
    }
}
template <typename T, int M>
hipError_t bwd_dh(int64_t Dh, const BwdParams& p, hipStream_t s) {
    switch (Dh) {
        case 16: return launch_bwd<T, M, 16>(p, s);
        case 32: return launch_bwd<T, M, 32>(p, s);
        case 64: return launch_bwd<T, M, 64>(p, s);
        default: return launch_bwd<T, M, 128>(p, s);
    }
}
template <typename T, int M>
hipError_t step_dh(int64_t Dh, const StepParams& p, hipStream_t s) {
    switch (Dh) {
        case 16: return launch_step<T, M, 16>(p, s);
        case 32: return launch_step<T, M, 32>(p, s);
        case 64: return launch_step<T, M, 64>(p, s);
        default: return launch_step<T, M, 128>(p, s);
    }
}

int hip_status(hipError_t e) { return e == hipSuccess ? ESA_OK : ESA_ERR_HIP; }

// Epochs tag the look-back words of one scan kernel launch.  The host counter is
// process-wide and only ever increments, so a workspace never sees the same host epoch twice
// within 2^29 launches; its start is drawn from the clock and the process id.
std::atomic<uint32_t> g_epoch{(uint32_t)(std::chrono::steady_clock::now().time_since_epoch().count() ^
                                         ((uint64_t)getpid() << 16))};

uint32_t next_epoch() { return g_epoch.fetch_add(1, std::memory_order_relaxed) & kHostEpochMask; }

// The epoch of a scan launch about to be enqueued on s.  Eager: the host counter.  While s is
// being recorded into a graph: the workspace's device epoch (header word 0), advanced by a
// one-thread kernel recorded just before the launch, so every replay tags its look-back words
// afresh.
int set_epoch(hipStream_t s, uint32_t* hdr, uint32_t* epoch, const uint32_t** word) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return ESA_ERR_HIP;
    if (cs == hipStreamCaptureStatusActive) {
        *epoch = 0;
        *word = hdr;
        return hip_status(launch_epoch_bump(hdr, s));
    }
    *epoch = next_epoch();
    *word = nullptr;
    return ESA_OK;
}

// The backward with optional gradient outputs: da, dv, dq all given (esa_scan_bwd) or all
// NULL (esa_scan_segment_bwd, which writes only the gradient reaching the initial state).
int scan_bwd_impl(bool grads, int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                  const void* gate_logit, const void* value, const void* query,
                  const float* init_state, const void* dy, const float* d_final_state,
                  const float* ckpt, void* d_gate_logit, void* d_value, void* d_query,
                  float* d_init_state, void* workspace, size_t workspace_bytes, void* stream) {
    Problem pr;
    int rc = check_sizes(B, T, H, Dh, dtype, mode, &pr);
    if (rc != ESA_OK) return rc;
    rc = check_test_flag(pr, grads);
    if (rc != ESA_OK) return rc;
    if (T > 0 && (!gate_logit || !value || !query || !dy)) return ESA_ERR_INVALID_ARG;
    if (grads ? (T > 0 && (!d_gate_logit || !d_value || !d_query))
              : (d_gate_logit || d_value || d_query || !d_init_state))
        return ESA_ERR_INVALID_ARG;
    const void* ptrs[] = {gate_logit, value, query, init_state, dy, d_final_state, ckpt,
                          d_gate_logit, d_value, d_query, d_init_state, workspace};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return ESA_ERR_INVALID_ARG;
    Layout L;
    rc = layout_of(pr, &L);
    if (rc != ESA_OK) return rc;
    const size_t seq = (size_t)(pr.nElem * pr.esize), st = (size_t)(pr.nLanes * 4);
    const size_t ckb = esa_scan_ckpt_bytes(B, T, H, Dh);
    const Range in[] = {{gate_logit, seq}, {value, seq}, {query, seq}, {init_state, st},
                        {dy, seq}, {d_final_state, st}, {ckpt, ckb}};
    const Range out[] = {{d_gate_logit, seq}, {d_value, seq}, {d_query, seq}, {d_init_state, st},
                         {workspace, workspace_bytes}};
    if (any_overlap(in, 7, out, 5)) return ESA_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < L.total)) return ESA_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (d_init_state) return hip_status(launch_copy_f32(d_init_state, d_final_state, pr.nLanes, s));
        return ESA_OK;
    }
    char* ws = static_cast<char*>(workspace);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(ws);
    uint64_t* fx = reinterpret_cast<uint64_t*>(ws + L.offX);
    uint64_t* fy = reinterpret_cast<uint64_t*>(ws + L.offY);
    const float* ck = ckpt;
    if (!ck) {
        // no checkpoint from the caller: one state-only forward pass into the workspace
        FwdParams f;
        memset(&f, 0, sizeof(f));
        f.a = gate_logit;
        f.v = value;
        f.e0 = init_state;
        f.ckpt = reinterpret_cast<float*>(ws + L.offCk);
        f.hdr = hdr;
        f.flagX = fx;
        f.flagY = fy;
        f.T = pr.T;
        f.C = pr.C;
        f.nLanes = pr.nLanes;
        f.nck = L.nck;
        f.nCB = L.nCB;
        f.nTiles = L.nTilesF;
        f.det = det_block(pr, L.nCB);
        f.withhold = 0;  // the checkpoint pass never takes the test instance
        rc = set_epoch(s, hdr, &f.epoch, &f.epochWord);
        if (rc != ESA_OK) return rc;
        rc = hip_status(ESA_DISPATCH(fwd, dtype, pr.mode, Dh, f, s));
        if (rc != ESA_OK) return rc;
        ck = f.ckpt;
    }
    BwdParams p;
    p.a = gate_logit;
    p.v = value;
    p.q = query;
    p.dy = dy;
    p.e0 = init_state;
    p.dET = d_final_state;
    p.ckpt = ck;
    p.da = d_gate_logit;
    p.dv = d_value;
    p.dq = d_query;
    p.de0 = d_init_state;
    p.hdr = hdr;
    p.flagX = fx;
    p.flagY = fy;
    p.T = pr.T;
    p.C = pr.C;
    p.nLanes = pr.nLanes;
    p.nck = L.nck;
    p.nCB = L.nCB;
    p.nTiles = L.nTilesB;
    p.det = det_block(pr, L.nCB);
    p.withhold = pr.forceTimeout;
    p.stats = pr.stats;
    rc = set_epoch(s, hdr, &p.epoch, &p.epochWord);
    if (rc != ESA_OK) return rc;
    return hip_status(ESA_DISPATCH(bwd, dtype, pr.mode, Dh, p, s));
}

}  // namespace

// ---------------------------------------------------------------------------------------
// The no-allocation forward (esa_scan_fwd_noalloc): its look-back words live in a static
// device array instead of a caller's workspace.  Each device that loads the library holds
// its own copy of the array until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory, so it is never passed to a kernel: at set-up (the
// first call on a device) hipGetSymbolAddress gives that device's address, which is kept per
// device and used everywhere the array's memory is needed.
// ---------------------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) uint8_t scratch[ESA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device: the device address of `scratch`, once set up

// The device address of this device's scratch array for a launch on stream s, set up on the
// first call on that device: the address is looked up with that device current, and the
// whole array is cleared once (a fill kernel on s; outside graph capture the call waits for
// it, so that later calls on other streams find it cleared).
int scratch_for(hipStream_t s, void** out) {
    int dev = 0;
    if (s) {
        if (hipStreamGetDevice(s, &dev) != hipSuccess) return ESA_ERR_HIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return ESA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return ESA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) {
        *out = g_scratch_ptr[dev];
        return ESA_OK;
    }
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return ESA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ESA_ERR_HIP;
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
    if (e != hipSuccess || !ptr) return ESA_ERR_HIP;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return ESA_ERR_HIP;
    if (launch_fill_zero(ptr, ESA_NOALLOC_SCRATCH_BYTES, s) != hipSuccess) return ESA_ERR_HIP;
    if (cs != hipStreamCaptureStatusActive && hipStreamSynchronize(s) != hipSuccess)
        return ESA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
    *out = ptr;
    return ESA_OK;
}

// The forward with fused readout.  `workspace` is the caller's (workspace_bytes long), or,
// with `noalloc`, NULL: the look-back words then live in this device's static scratch array.
int scan_fwd_impl(bool noalloc, int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                  const void* gate_logit, const void* value, const void* query,
                  const float* init_state, void* y, float* final_state, float* ckpt,
                  void* workspace, size_t workspace_bytes, void* stream) {
    Problem pr;
    int rc = check_sizes(B, T, H, Dh, dtype, mode, &pr);
    if (rc != ESA_OK) return rc;
    rc = check_test_flag(pr, !noalloc);
    if (rc != ESA_OK) return rc;
    if (T > 0 && (!gate_logit || !value || !query || !y)) return ESA_ERR_INVALID_ARG;
    const void* ptrs[] = {gate_logit, value, query, init_state, y, final_state, ckpt, workspace};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return ESA_ERR_INVALID_ARG;
    Layout L;
    rc = layout_of(pr, &L);
    if (rc != ESA_OK) return rc;
    const size_t seq = (size_t)(pr.nElem * pr.esize), st = (size_t)(pr.nLanes * 4);
    const size_t ckb = esa_scan_ckpt_bytes(B, T, H, Dh);
    const Range in[] = {{gate_logit, seq}, {value, seq}, {query, seq},
                        {init_state == final_state ? nullptr : init_state, st}};
    const Range out[] = {{y, seq}, {final_state, st}, {ckpt, ckb}, {workspace, workspace_bytes}};
    if (any_overlap(in, 4, out, 4)) return ESA_ERR_INVALID_ARG;
    // look-back words of the forward alone: header, X and Y over the forward's tiles
    const size_t xbytes = align256((size_t)L.nTilesFV * (size_t)pr.nLanes * 8);
    size_t offY = L.offY;
    if (noalloc) {
        if (T > 0 && 256 + 2 * xbytes > (size_t)ESA_NOALLOC_SCRATCH_BYTES) return ESA_ERR_SCRATCH_LIMIT;
        offY = 256 + xbytes;
    } else if (T > 0 && (!workspace || workspace_bytes < L.total)) {
        return ESA_ERR_WORKSPACE;
    }

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {
        if (final_state && final_state != init_state)
            return hip_status(launch_copy_f32(final_state, init_state, pr.nLanes, s));
        return ESA_OK;
    }
    if (noalloc) {
        rc = scratch_for(s, &workspace);
        if (rc != ESA_OK) return rc;
    }
    char* ws = static_cast<char*>(workspace);
    FwdParams p;
    p.a = gate_logit;
    p.v = value;
    p.q = query;
    p.e0 = init_state;
    p.y = y;
    p.eT = final_state;
    p.ckpt = ckpt;
    p.prod = nullptr;
    p.hdr = reinterpret_cast<uint32_t*>(ws);
    p.flagX = reinterpret_cast<uint64_t*>(ws + L.offX);
    p.flagY = reinterpret_cast<uint64_t*>(ws + offY);
    p.T = pr.T;
    p.C = pr.C;
    p.nLanes = pr.nLanes;
    p.nck = L.nck;
    p.nCB = L.nCB;
    p.nTiles = L.nTilesFV;
    p.det = det_block(pr, L.nCB);
    p.withhold = pr.forceTimeout;
    p.stats = pr.stats;
    p.variant = L.fwdVariant;
    rc = set_epoch(s, p.hdr, &p.epoch, &p.epochWord);
    if (rc != ESA_OK) return rc;
    return hip_status(ESA_DISPATCH(fwd, dtype, pr.mode, Dh, p, s));
}

}  // namespace

extern "C" {

int esa_scan_fwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                 const void* gate_logit, const void* value, const void* query,
                 const float* init_state, void* y, float* final_state, float* ckpt,
                 void* workspace, size_t workspace_bytes, void* stream) {
    return scan_fwd_impl(false, B, T, H, Dh, dtype, mode, gate_logit, value, query, init_state, y,
                         final_state, ckpt, workspace, workspace_bytes, stream);
}

int esa_scan_fwd_noalloc(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void* gate_logit, const void* value, const void* query,
                         const float* init_state, void* y, float* final_state, float* ckpt,
                         void* stream) {
    return scan_fwd_impl(true, B, T, H, Dh, dtype, mode, gate_logit, value, query, init_state, y,
                         final_state, ckpt, nullptr, 0, stream);
}


int esa_abi_version(void) { return ESA_ABI_VERSION; }

const char* esa_status_string(int status) {
    switch (status) {
        case ESA_OK: return "ESA_OK: success";
        case ESA_ERR_INVALID_ARG:
            return "ESA_ERR_INVALID_ARG: null pointer, bad size or enum, misaligned or overlapping buffer";
        case ESA_ERR_UNSUPPORTED: return "ESA_ERR_UNSUPPORTED: Dh not in {16, 32, 64, 128} or problem too large";
        case ESA_ERR_WORKSPACE: return "ESA_ERR_WORKSPACE: workspace missing or smaller than esa_scan_workspace_bytes()";
        case ESA_ERR_HIP: return "ESA_ERR_HIP: the HIP runtime rejected a kernel launch";
        case ESA_ERR_TIMEOUT:
            return "ESA_ERR_TIMEOUT: a cross-tile wait of a scan on this workspace timed out; "
                   "the outputs that depend on it are NaN";
        case ESA_ERR_SCRATCH_LIMIT:
            return "ESA_ERR_SCRATCH_LIMIT: the problem needs more look-back scratch than the "
                   "no-allocation forward's static array holds (ESA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown esa_status";
    }
}

size_t esa_scan_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype) {
    Problem pr;
    if (check_sizes(B, T, H, Dh, dtype, ESA_DIRECT, &pr) != ESA_OK) return 0;
    Layout L;
    if (layout_of(pr, &L) != ESA_OK) return 0;
    return L.total;
}

size_t esa_scan_ckpt_bytes(int64_t B, int64_t T, int64_t H, int64_t Dh) {
    Problem pr;
    if (check_sizes(B, T, H, Dh, ESA_F32, ESA_DIRECT, &pr) != ESA_OK) return 0;
    int64_t n;
    if (!mul64(cdiv(T, kCkptChunk), pr.nLanes, &n) || !mul64(n, 4, &n)) return 0;
    return (size_t)n;
}

int esa_workspace_status(const void* workspace, uint32_t* info, void* stream) {
    if (!info || (workspace && !aligned16(workspace))) return ESA_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return ESA_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) return ESA_ERR_INVALID_ARG;  // it waits for the stream
    const void* src = workspace;
    if (!src) {  // this device's no-allocation scratch, if a call has set it up
        int dev = 0;
        if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
            return ESA_ERR_HIP;
        if (dev < 0 || dev >= kMaxDevices) return ESA_ERR_UNSUPPORTED;
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        src = g_scratch_ptr[dev];
    }
    uint32_t h[64] = {0};
    if (src) {
        if (hipMemcpyAsync(h, src, sizeof(h), hipMemcpyDeviceToHost, s) != hipSuccess ||
            hipStreamSynchronize(s) != hipSuccess)
            return ESA_ERR_HIP;
    }
    uint32_t sum[kStatWords] = {0};
    for (int x = 0; x < 8; ++x)
        for (int k = 0; k < kStatWords; ++k) {
            const uint32_t v = h[kStatWordsOffset + x * kStatWords + k];
            if (k == kStatMaxWalk)
                sum[k] = v > sum[k] ? v : sum[k];
            else
                sum[k] += v;
        }
    info[0] = h[3];
    for (int k = 0; k < kStatWords; ++k) info[1 + k] = sum[k];
    return h[3] ? ESA_ERR_TIMEOUT : ESA_OK;
}

int esa_workspace_init(void* workspace, size_t bytes, void* stream) {
    if (!workspace || !aligned16(workspace)) return ESA_ERR_INVALID_ARG;
    return hip_status(launch_fill_zero(workspace, bytes, (hipStream_t)stream));
}

int esa_scan_bwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                 const void* gate_logit, const void* value, const void* query,
                 const float* init_state, const void* dy, const float* d_final_state,
                 const float* ckpt, void* d_gate_logit, void* d_value, void* d_query,
                 float* d_init_state, void* workspace, size_t workspace_bytes, void* stream) {
    return scan_bwd_impl(true, B, T, H, Dh, dtype, mode, gate_logit, value, query, init_state, dy,
                         d_final_state, ckpt, d_gate_logit, d_value, d_query, d_init_state,
                         workspace, workspace_bytes, stream);
}

int esa_state_step(int64_t B, int64_t H, int64_t Dh, int dtype, int mode, const void* gate_logit,
                   const void* value, const void* query, float* state, void* y, void* stream) {
    Problem pr;
    int rc = check_sizes(B, 1, H, Dh, dtype, mode, &pr);
    if (rc != ESA_OK) return rc;
    rc = check_test_flag(pr, false);
    if (rc != ESA_OK) return rc;
    if (!gate_logit || !value || !query || !state || !y) return ESA_ERR_INVALID_ARG;
    const void* ptrs[] = {gate_logit, value, query, state, y};
    for (const void* q : ptrs)
        if (!aligned16(q)) return ESA_ERR_INVALID_ARG;
    const size_t tok = (size_t)(pr.nLanes * pr.esize), st = (size_t)(pr.nLanes * 4);
    const Range in[] = {{gate_logit, tok}, {value, tok}, {query, tok}};
    const Range out[] = {{state, st}, {y, tok}};
    if (any_overlap(in, 3, out, 2)) return ESA_ERR_INVALID_ARG;
    StepParams p;
    p.a = gate_logit;
    p.v = value;
    p.q = query;
    p.state = state;
    p.y = y;
    p.nLanes = pr.nLanes;
    return hip_status(ESA_DISPATCH(step, dtype, pr.mode, Dh, p, (hipStream_t)stream));
}

int esa_scan_segment_fwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void* gate_logit, const void* value, float* seg_state,
                         float* seg_gate_prod, void* workspace, size_t workspace_bytes,
                         void* stream) {
    Problem pr;
    int rc = check_sizes(B, T, H, Dh, dtype, mode, &pr);
    if (rc != ESA_OK) return rc;
    rc = check_test_flag(pr, false);
    if (rc != ESA_OK) return rc;
    if (!seg_state || !seg_gate_prod) return ESA_ERR_INVALID_ARG;
    if (T > 0 && (!gate_logit || !value)) return ESA_ERR_INVALID_ARG;
    const void* ptrs[] = {gate_logit, value, seg_state, seg_gate_prod, workspace};
    for (const void* q : ptrs)
        if (q && !aligned16(q)) return ESA_ERR_INVALID_ARG;
    Layout L;
    rc = layout_of(pr, &L);
    if (rc != ESA_OK) return rc;
    const size_t seq = (size_t)(pr.nElem * pr.esize), st = (size_t)(pr.nLanes * 4);
    const Range in[] = {{gate_logit, seq}, {value, seq}};
    const Range out[] = {{seg_state, st}, {seg_gate_prod, st}, {workspace, workspace_bytes}};
    if (any_overlap(in, 2, out, 3)) return ESA_ERR_INVALID_ARG;
    if (T > 0 && (!workspace || workspace_bytes < L.total)) return ESA_ERR_WORKSPACE;

    hipStream_t s = (hipStream_t)stream;
    if (T == 0) {  // the identity pair: zero state, unit product
        rc = hip_status(launch_fill_f32(seg_state, 0.0f, pr.nLanes, s));
        if (rc != ESA_OK) return rc;
        return hip_status(launch_fill_f32(seg_gate_prod, 1.0f, pr.nLanes, s));
    }
    char* ws = static_cast<char*>(workspace);
    FwdParams f;
    memset(&f, 0, sizeof(f));
    f.a = gate_logit;
    f.v = value;
    f.eT = seg_state;
    f.prod = seg_gate_prod;
    f.hdr = reinterpret_cast<uint32_t*>(ws);
    f.flagX = reinterpret_cast<uint64_t*>(ws + L.offX);
    f.flagY = reinterpret_cast<uint64_t*>(ws + L.offY);
    f.T = pr.T;
    f.C = pr.C;
    f.nLanes = pr.nLanes;
    f.nck = L.nck;
    f.nCB = L.nCB;
    f.nTiles = L.nTilesF;
    f.det = det_block(pr, L.nCB);
    f.withhold = 0;
    rc = set_epoch(s, f.hdr, &f.epoch, &f.epochWord);
    if (rc != ESA_OK) return rc;
    return hip_status(ESA_DISPATCH(fwd, dtype, pr.mode, Dh, f, s));
}

int esa_scan_segment_bwd(int64_t B, int64_t T, int64_t H, int64_t Dh, int dtype, int mode,
                         const void* gate_logit, const void* value, const void* query,
                         const float* init_state, const void* dy, const float* ckpt,
                         float* seg_d_init, void* workspace, size_t workspace_bytes,
                         void* stream) {
    return scan_bwd_impl(false, B, T, H, Dh, dtype, mode, gate_logit, value, query, init_state, dy,
                         nullptr, ckpt, nullptr, nullptr, nullptr, seg_d_init, workspace,
                         workspace_bytes, stream);
}

int esa_segment_compose(int64_t nseg, int64_t nLanes, int reverse, const float* seg_gate_prod,
                        const float* seg_agg, const float* boundary, float* carry, float* total,
                        void* stream) {
    if (nseg < 1 || nLanes < 1 || (reverse != 0 && reverse != 1)) return ESA_ERR_INVALID_ARG;
    if (!seg_gate_prod || !seg_agg || !carry) return ESA_ERR_INVALID_ARG;
    int64_t n, bytes;
    if (!mul64(nseg, nLanes, &n) || !mul64(n, 4, &bytes)) return ESA_ERR_INVALID_ARG;
    const void* ptrs[] = {seg_gate_prod, seg_agg, boundary, carry, total};
    for (const void* q : ptrs)
        if (q && (reinterpret_cast<uintptr_t>(q) & 3u)) return ESA_ERR_INVALID_ARG;
    const Range in[] = {{seg_gate_prod, (size_t)bytes}, {seg_agg, (size_t)bytes},
                        {boundary, (size_t)nLanes * 4}};
    const Range out[] = {{carry, (size_t)bytes}, {total, (size_t)nLanes * 4}};
    if (any_overlap(in, 3, out, 2)) return ESA_ERR_INVALID_ARG;
    return hip_status(launch_compose(nseg, nLanes, reverse, seg_gate_prod, seg_agg, boundary,
                                     carry, total, (hipStream_t)stream));
}

}  // extern "C"
